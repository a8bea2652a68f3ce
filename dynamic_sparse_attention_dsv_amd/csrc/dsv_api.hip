// C ABI of libdsv: argument validation, workspace carving and launch sequencing.
// The declarations and the contract of every entry point are in include/dsv.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dsv.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

dsv_status fail(dsv_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

constexpr size_t kWsAlign = 256;
size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct Prob {
  int b, h, n, d, bq, bk, k, r, dtype;
  float sm, ps;
  int bh() const { return b * h; }
  int nqb() const { return n / bq; }
  int nkb() const { return n / bk; }
  size_t esize() const { return dtype == DSV_BF16 ? 2 : 4; }
  size_t tensor_elems() const { return (size_t)b * h * n * d; }
};

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Common checks; `need_rank` for the predictor, `need_k` for selection and attention.
dsv_status to_prob(const dsv_problem* p, Prob& o, bool need_rank) {
  if (!p) return fail(DSV_ERR_INVALID_ARGUMENT, "problem pointer is NULL");
  o = Prob{p->batch, p->heads, p->seq_len, p->head_dim, p->q_block, p->kv_block, p->topk, p->rank, p->dtype,
           p->sm_scale, p->pred_scale};
  char buf[256];
  if (o.b < 1 || o.h < 1 || o.n < 1 || o.d < 1 || o.bq < 1 || o.bk < 1) {
    snprintf(buf, sizeof buf, "sizes must be positive (B=%d H=%d N=%d d=%d Bq=%d Bk=%d)", o.b, o.h, o.n, o.d, o.bq,
             o.bk);
    return fail(DSV_ERR_INVALID_ARGUMENT, buf);
  }
  if (o.n % o.bq || o.n % o.bk || o.bq % o.bk) {
    snprintf(buf, sizeof buf, "N=%d must be a multiple of Bq=%d and Bk=%d, and Bq of Bk", o.n, o.bq, o.bk);
    return fail(DSV_ERR_INVALID_ARGUMENT, buf);
  }
  if (o.k < 1 || o.k > o.nkb()) {
    snprintf(buf, sizeof buf, "topk=%d out of range [1, N/Bk=%d]", o.k, o.nkb());
    return fail(DSV_ERR_INVALID_ARGUMENT, buf);
  }
  if (o.dtype != DSV_F32 && o.dtype != DSV_BF16) return fail(DSV_ERR_INVALID_ARGUMENT, "dtype must be DSV_F32 or DSV_BF16");
  if (need_rank && o.r < 1) return fail(DSV_ERR_INVALID_ARGUMENT, "rank must be positive");
  if (!std::isfinite(o.sm) || !std::isfinite(o.ps)) return fail(DSV_ERR_INVALID_ARGUMENT, "scales must be finite");
  if (o.sm <= 0.f) o.sm = 1.f / std::sqrt((float)o.d);
  if (o.ps <= 0.f) o.ps = 1.f / std::sqrt((float)o.d);
  if ((double)o.b * o.h * o.n * (o.d > o.r ? o.d : o.r) >= 2147483648.0 * 16)
    return fail(DSV_ERR_UNSUPPORTED, "tensor too large");
  if ((double)o.b * o.h * o.nqb() >= 2147483647.0 || (double)o.b * o.h * o.nkb() >= 2147483647.0)
    return fail(DSV_ERR_UNSUPPORTED, "too many blocks");
  if (o.nkb() > 4096) return fail(DSV_ERR_UNSUPPORTED, "N/Bk must be <= 4096");
  return DSV_OK;
}

dsv_status check_bf16_attn(const Prob& o) {
  if (o.dtype != DSV_BF16) return DSV_OK;
  char buf[200];
  if ((o.d != 64 && o.d != 128) || (o.bq != 64 && o.bq != 128) || o.bk != 64) {
    snprintf(buf, sizeof buf, "bf16 instances need d in {64,128}, Bq in {64,128}, Bk = 64 (got d=%d Bq=%d Bk=%d)",
             o.d, o.bq, o.bk);
    return fail(DSV_ERR_UNSUPPORTED, buf);
  }
  return DSV_OK;
}

dsv_status check_f32_attn(const Prob& o) {
  if (o.dtype == DSV_F32 && o.d > 128) return fail(DSV_ERR_UNSUPPORTED, "f32 instances need d <= 128");
  return DSV_OK;
}

dsv_status check_ptr(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(DSV_ERR_INVALID_ARGUMENT, std::string(name) + " is NULL");
  if (!aligned(p, align))
    return fail(DSV_ERR_INVALID_ARGUMENT, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return DSV_OK;
}

// The optional rounding residual of O: bf16 problems only, 16-byte aligned when given.
dsv_status check_residual(const Prob& o, const void* o_lo) {
  if (!o_lo) return DSV_OK;
  if (o.dtype != DSV_BF16) return fail(DSV_ERR_INVALID_ARGUMENT, "o_lo must be NULL for float32 problems");
  return check_ptr(o_lo, "o_lo");
}

dsv_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return DSV_OK;
  return fail(DSV_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define TRY(x)                      \
  do {                              \
    dsv_status s_ = (x);            \
    if (s_ != DSV_OK) return s_;    \
  } while (0)

// Optional per-launch timing (dsv_timing_begin / dsv_timing_end): when enabled on
// this thread, every launch is bracketed by two HIP events on its stream.
struct TimingRec {
  const char* name;
  hipEvent_t start, stop;
};
thread_local bool g_timing = false;
thread_local std::vector<TimingRec> g_recs;

template <class F>
dsv_status timed(const char* name, hipStream_t st, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  const bool on = g_timing && hipEventCreate(&a) == hipSuccess && hipEventCreate(&b) == hipSuccess;
  if (on) (void)hipEventRecord(a, st);
  const hipError_t e = launch();
  if (on) {
    (void)hipEventRecord(b, st);
    g_recs.push_back({name, a, b});
  } else {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
  return hip_status(e, name);
}
#define TRY_HIP(x, name) TRY(timed(name, st, [&] { return (x); }))

// The opt-in device check of the block lists (DSV_DEBUG_VALIDATE=1, read at each call).
bool debug_validate() {
  const char* v = std::getenv("DSV_DEBUG_VALIDATE");
  return v && std::strcmp(v, "1") == 0;
}

dsv_status check_lists(const Prob& o, const int32_t* block_idx, const int32_t* block_counts, hipStream_t st) {
  if (!debug_validate()) return DSV_OK;
  uint32_t bad = 0;
  TRY(hip_status(dsv::check_block_lists(block_idx, block_counts, o.bh() * o.nqb(), o.nkb(), o.k, st, &bad),
                 "DSV_DEBUG_VALIDATE list check"));
  if (bad)
    return fail(DSV_ERR_INVALID_ARGUMENT, "DSV_DEBUG_VALIDATE: " + std::to_string(bad) +
                                              " query block(s) use block indices that are out of range or repeated");
  return DSV_OK;
}

// ---------------------------------------------------------------- workspace layouts

struct PredictWs {
  size_t qlr, klr, scratch, lse, scores, total;
};
PredictWs predict_ws(const Prob& o) {
  PredictWs w{};
  const size_t lr = align_up((size_t)o.bh() * o.n * o.r * o.esize());
  w.qlr = 0;
  w.klr = lr;
  size_t off = 2 * lr;
  if (o.dtype == DSV_BF16) {
    w.scratch = off;
    off += align_up(dsv::score_scratch_bytes(o.bh() * (o.n / 256), o.nkb()));
  } else {
    w.lse = off;
    off += align_up((size_t)o.bh() * o.n * sizeof(float));
    w.scores = off;  // the fused representative call's scores before its selection (fp32 path)
    off += align_up((size_t)o.bh() * o.nqb() * o.nkb() * sizeof(float));
  }
  w.total = off;
  return w;
}

struct BwdWs {
  size_t dvec, lse2, dvec_s, bitmap, counts, col_ptr, rows, order, f16, total;
};
BwdWs bwd_ws(const Prob& o) {
  BwdWs w{};
  size_t off = 0;
  const size_t rowf = align_up((size_t)o.bh() * o.n * sizeof(float));
  if (o.dtype == DSV_BF16) {
    w.lse2 = off; off += rowf;
    w.dvec_s = off; off += rowf;
    w.order = off; off += align_up((size_t)o.bh() * o.nkb() * 4);
    w.f16 = off; off += align_up(dsv::bwd_f16_ws_bytes(o.bh(), o.n, o.d));
  }
  w.dvec = off; off += rowf;
  const int words = (o.nqb() + 31) / 32;
  w.bitmap = off; off += align_up((size_t)o.bh() * o.nkb() * words * 4);
  w.counts = off; off += align_up((size_t)o.bh() * o.nkb() * 4);
  w.col_ptr = off; off += align_up((size_t)o.bh() * (o.nkb() + 1) * 4);
  w.rows = off; off += align_up((size_t)o.bh() * o.nqb() * o.k * 4);
  w.total = off;
  return w;
}

// the bf16 training forward (o_lo requested) needs scratch; the inference forward and fp32 none
size_t fwd_ws_bytes(const Prob& o) {
  return o.dtype == DSV_BF16 ? dsv::attn_fwd_bf16_ws_bytes(o.bh(), o.n, o.d) : 0;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

const char* dsv_status_string(dsv_status s) {
  switch (s) {
    case DSV_OK: return "DSV_OK";
    case DSV_ERR_INVALID_ARGUMENT: return "DSV_ERR_INVALID_ARGUMENT";
    case DSV_ERR_UNSUPPORTED: return "DSV_ERR_UNSUPPORTED";
    case DSV_ERR_WORKSPACE_TOO_SMALL: return "DSV_ERR_WORKSPACE_TOO_SMALL";
    case DSV_ERR_HIP: return "DSV_ERR_HIP";
  }
  return "DSV_ERR_UNKNOWN";
}

const char* dsv_last_error(void) { return g_err.c_str(); }

int32_t dsv_version(void) { return 100; }

size_t dsv_peak_probe_workspace_size(int32_t kind) {
  const size_t per_thread = (size_t)dsv::kProbeMaxCus * 8 * 256 * sizeof(float);  // one word per probe thread
  if (kind == DSV_PEAK_MFMA_BF16 || kind == DSV_PEAK_MFMA_F16 || kind == DSV_PEAK_EXP_F32) return per_thread;
  if (kind == DSV_PEAK_HBM_COPY) return dsv::kProbeCopyBytes;
  if (kind == DSV_PEAK_HBM_READ) return dsv::kProbeCopyBytes + per_thread;
  return 0;
}

dsv_status dsv_peak_probe(int32_t kind, int32_t repeats, void* workspace, size_t workspace_bytes, double* rate,
                          void* stream) {
  g_err.clear();
  const size_t need = dsv_peak_probe_workspace_size(kind);
  if (need == 0) return fail(DSV_ERR_INVALID_ARGUMENT, "unknown probe kind " + std::to_string(kind));
  if (repeats < 1 || repeats > 100) return fail(DSV_ERR_INVALID_ARGUMENT, "repeats must lie in [1, 100]");
  if (!rate) return fail(DSV_ERR_INVALID_ARGUMENT, "rate is null");
  TRY(check_ptr(workspace, "workspace", kWsAlign));
  if (workspace_bytes < need)
    return fail(DSV_ERR_WORKSPACE_TOO_SMALL, "probe workspace needs " + std::to_string(need) + " bytes");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
    if (a) (void)hipEventDestroy(a);
    return fail(DSV_ERR_HIP, "hipEventCreate failed");
  }
  double best_ms = 0.0, work = 0.0;
  dsv_status s = DSV_OK;
  for (int i = 0; i < repeats && s == DSV_OK; ++i) {
    float ms = 0.f;
    hipError_t e = hipEventRecord(a, st);
    if (e == hipSuccess) e = dsv::launch_peak_probe(kind, workspace, need, st, &work);
    if (e == hipSuccess) e = hipEventRecord(b, st);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e != hipSuccess) s = hip_status(e, "peak probe");
    else if (i == 0 || ms < best_ms) best_ms = ms;
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (s != DSV_OK) return s;
  if (!(best_ms > 0.0)) return fail(DSV_ERR_HIP, "peak probe: no elapsed time recorded");
  *rate = work / (best_ms * 1e-3);
  return DSV_OK;
}

dsv_status dsv_timing_begin(void) {
  g_err.clear();
  if (g_timing) return fail(DSV_ERR_INVALID_ARGUMENT, "timing already active on this thread");
  g_recs.clear();
  g_timing = true;
  return DSV_OK;
}

int32_t dsv_timing_end(dsv_kernel_stat* out, int32_t capacity) {
  g_timing = false;
  std::vector<dsv_kernel_stat> agg;
  for (const TimingRec& r : g_recs) {
    float ms = 0.f;
    const bool ok = hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess;
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
    if (!ok) continue;
    dsv_kernel_stat* a = nullptr;
    for (auto& x : agg)
      if (std::strncmp(x.name, r.name, sizeof x.name) == 0) a = &x;
    if (!a) {
      agg.push_back({});
      a = &agg.back();
      std::strncpy(a->name, r.name, sizeof a->name - 1);
      a->min_ms = ms;
      a->max_ms = ms;
    }
    a->launches += 1;
    a->total_ms += ms;
    a->min_ms = ms < a->min_ms ? ms : a->min_ms;
    a->max_ms = ms > a->max_ms ? ms : a->max_ms;
  }
  g_recs.clear();
  const int32_t n = (int32_t)agg.size();
  for (int32_t i = 0; out && i < n && i < capacity; ++i) out[i] = agg[i];
  return n;
}

size_t dsv_predict_workspace_size(const dsv_problem* p) {
  Prob o;
  if (to_prob(p, o, true) != DSV_OK) return 0;
  return predict_ws(o).total;
}

namespace {
// shared by dsv_predict (rep < 0) and dsv_predict_representative (rep = the representative row)
dsv_status predict_impl(const dsv_problem* p, const void* q, const void* k, const void* wq, const void* wk,
                        void* workspace, size_t workspace_bytes, float* block_scores, int rep, void* stream) {
  Prob o;
  TRY(to_prob(p, o, true));
  if (rep >= o.bq) return fail(DSV_ERR_INVALID_ARGUMENT, "rep_row must lie in [0, q_block)");
  if (o.dtype == DSV_BF16) {
    if ((o.d != 64 && o.d != 128) || (o.r != 16 && o.r != 32) || (o.bq != 64 && o.bq != 128) || o.bk != 64 ||
        o.n % 256)
      return fail(DSV_ERR_UNSUPPORTED, "bf16 predictor needs d in {64,128}, r in {16,32}, Bq in {64,128}, Bk = 64, N % 256 == 0");
  } else if (o.r > 64) {
    return fail(DSV_ERR_UNSUPPORTED, "f32 predictor needs r <= 64");
  }
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(wq, "wq", o.dtype == DSV_BF16 ? 2 : 4));
  TRY(check_ptr(wk, "wk", o.dtype == DSV_BF16 ? 2 : 4));
  TRY(check_ptr(block_scores, "block_scores"));
  TRY(check_ptr(workspace, "workspace", kWsAlign));
  const PredictWs w = predict_ws(o);
  if (workspace_bytes < w.total)
    return fail(DSV_ERR_WORKSPACE_TOO_SMALL, "predict workspace needs " + std::to_string(w.total) + " bytes");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The query projection carries the logit scale in base-2 units, applied before its one rounding:
  // Q~ = rho(pred_scale log2(e) Q Wq), so <Q~_i, K_lr_j> is the logit l_ij / ln 2 and the score
  // kernels take 2^<Q~_i, K_lr_j> (the fp32 kernels as exp(ln 2 <Q~_i, K_lr_j>)).
  const float q_scale = o.ps * 1.4426950408889634f;  // log2(e)
  if (o.dtype == DSV_BF16) {
    uint16_t* qlr = at<uint16_t>(workspace, w.qlr);
    uint16_t* klr = at<uint16_t>(workspace, w.klr);
    TRY_HIP(dsv::launch_proj_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(wq), qlr, o.bh(), o.n,
                                  o.h, o.d, o.r, q_scale, st), "proj_kernel(q)");
    TRY_HIP(dsv::launch_proj_bf16(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(wk), klr, o.bh(), o.n,
                                  o.h, o.d, o.r, 1.f, st), "proj_kernel(k)");
    TRY_HIP(dsv::launch_scores_bf16(qlr, klr, at<float>(workspace, w.scratch), block_scores, o.bh(), o.n, o.nkb(),
                                    o.r, o.bq, rep, st), "scores_kernel");
  } else {
    float* qlr = at<float>(workspace, w.qlr);
    float* klr = at<float>(workspace, w.klr);
    TRY_HIP(dsv::launch_proj_f32(static_cast<const float*>(q), static_cast<const float*>(wq), qlr, o.bh(), o.n, o.h,
                                 o.d, o.r, q_scale, st), "proj_kernel(q)");
    TRY_HIP(dsv::launch_proj_f32(static_cast<const float*>(k), static_cast<const float*>(wk), klr, o.bh(), o.n, o.h,
                                 o.d, o.r, 1.f, st), "proj_kernel(k)");
    if (rep < 0)
      TRY_HIP(dsv::launch_scores_f32(qlr, klr, at<float>(workspace, w.lse), block_scores, o.bh(), o.n, o.r, o.bq,
                                     o.bk, 0.6931471805599453f /* ln 2 */, st), "scores_kernel");
    else
      TRY_HIP(dsv::launch_rep_scores_f32(qlr, klr, at<float>(workspace, w.lse), block_scores, o.bh(), o.n, o.r,
                                         o.bq, o.bk, 0.6931471805599453f /* ln 2 */, rep, st), "scores_kernel");
  }
  return DSV_OK;
}
}  // namespace

dsv_status dsv_predict(const dsv_problem* p, const void* q, const void* k, const void* wq, const void* wk,
                       void* workspace, size_t workspace_bytes, float* block_scores, void* stream) {
  g_err.clear();
  return predict_impl(p, q, k, wq, wk, workspace, workspace_bytes, block_scores, -1, stream);
}

dsv_status dsv_predict_representative(const dsv_problem* p, const void* q, const void* k, const void* wq,
                                      const void* wk, int32_t rep_row, void* workspace, size_t workspace_bytes,
                                      float* block_scores, void* stream) {
  g_err.clear();
  if (rep_row < 0) return fail(DSV_ERR_INVALID_ARGUMENT, "rep_row must lie in [0, q_block)");
  return predict_impl(p, q, k, wq, wk, workspace, workspace_bytes, block_scores, rep_row, stream);
}

dsv_status dsv_predict_select_representative(const dsv_problem* p, const void* q, const void* k, const void* wq,
                                             const void* wk, int32_t rep_row, void* workspace, size_t workspace_bytes,
                                             int32_t* block_idx, void* stream) {
  g_err.clear();
  Prob o;
  TRY(to_prob(p, o, true));
  if (rep_row < 0 || rep_row >= o.bq) return fail(DSV_ERR_INVALID_ARGUMENT, "rep_row must lie in [0, q_block)");
  if (o.dtype == DSV_BF16) {
    if ((o.d != 64 && o.d != 128) || (o.r != 16 && o.r != 32) || (o.bq != 64 && o.bq != 128) || o.bk != 64 ||
        o.n % 256)
      return fail(DSV_ERR_UNSUPPORTED, "bf16 predictor needs d in {64,128}, r in {16,32}, Bq in {64,128}, Bk = 64, N % 256 == 0");
  } else if (o.r > 64) {
    return fail(DSV_ERR_UNSUPPORTED, "f32 predictor needs r <= 64");
  }
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(wq, "wq", o.dtype == DSV_BF16 ? 2 : 4));
  TRY(check_ptr(wk, "wk", o.dtype == DSV_BF16 ? 2 : 4));
  TRY(check_ptr(block_idx, "block_idx", 4));
  TRY(check_ptr(workspace, "workspace", kWsAlign));
  const PredictWs w = predict_ws(o);
  if (workspace_bytes < w.total)
    return fail(DSV_ERR_WORKSPACE_TOO_SMALL, "predict workspace needs " + std::to_string(w.total) + " bytes");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float q_scale = o.ps * 1.4426950408889634f;  // log2(e): Q~ carries the logit scale (as dsv_predict)
  if (o.dtype == DSV_BF16) {
    uint16_t* qlr = at<uint16_t>(workspace, w.qlr);
    uint16_t* klr = at<uint16_t>(workspace, w.klr);
    TRY_HIP(dsv::launch_proj_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(wq), qlr, o.bh(), o.n,
                                  o.h, o.d, o.r, q_scale, st), "proj_kernel(q)");
    TRY_HIP(dsv::launch_proj_bf16(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(wk), klr, o.bh(), o.n,
                                  o.h, o.d, o.r, 1.f, st), "proj_kernel(k)");
    TRY_HIP(dsv::launch_rep_select_bf16(qlr, klr, at<float>(workspace, w.scratch), block_idx, o.bh(), o.n, o.nkb(),
                                        o.r, o.bq, rep_row, o.k, st), "rep_select_kernel");
  } else {  // the plain VALU path for small fp32 problems: scores into the workspace, then top-k
    float* qlr = at<float>(workspace, w.qlr);
    float* klr = at<float>(workspace, w.klr);
    float* sc = at<float>(workspace, w.scores);
    TRY_HIP(dsv::launch_proj_f32(static_cast<const float*>(q), static_cast<const float*>(wq), qlr, o.bh(), o.n, o.h,
                                 o.d, o.r, q_scale, st), "proj_kernel(q)");
    TRY_HIP(dsv::launch_proj_f32(static_cast<const float*>(k), static_cast<const float*>(wk), klr, o.bh(), o.n, o.h,
                                 o.d, o.r, 1.f, st), "proj_kernel(k)");
    TRY_HIP(dsv::launch_rep_scores_f32(qlr, klr, at<float>(workspace, w.lse), sc, o.bh(), o.n, o.r, o.bq, o.bk,
                                       0.6931471805599453f /* ln 2 */, rep_row, st), "scores_kernel");
    TRY_HIP(dsv::launch_select_topk(sc, block_idx, o.bh() * o.nqb(), o.nkb(), o.k, st), "select_topk_kernel");
  }
  return DSV_OK;
}

dsv_status dsv_select_topk(const dsv_problem* p, const float* block_scores, int32_t* block_idx, void* stream) {
  g_err.clear();
  Prob o;
  TRY(to_prob(p, o, false));
  TRY(check_ptr(block_scores, "block_scores", 4));
  TRY(check_ptr(block_idx, "block_idx", 4));
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY_HIP(dsv::launch_select_topk(block_scores, block_idx, o.bh() * o.nqb(), o.nkb(), o.k, st), "select_topk_kernel");
  return DSV_OK;
}

dsv_status dsv_select_mass(const dsv_problem* p, const float* block_scores, float tau, int32_t* block_idx,
                           int32_t* block_counts, void* stream) {
  g_err.clear();
  Prob o;
  TRY(to_prob(p, o, false));
  TRY(check_ptr(block_scores, "block_scores", 4));
  TRY(check_ptr(block_idx, "block_idx", 4));
  TRY(check_ptr(block_counts, "block_counts", 4));
  if (!(tau > 0.f && tau <= 1.f)) return fail(DSV_ERR_INVALID_ARGUMENT, "tau must lie in (0, 1]");
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY_HIP(dsv::launch_select_mass(block_scores, block_idx, block_counts, o.bh() * o.nqb(), o.nkb(), o.k, tau, st),
          "select_mass_kernel");
  return DSV_OK;
}

dsv_status dsv_head_density(const dsv_problem* p, const int32_t* block_counts, float dense_above, float* density,
                            int32_t* dense, void* stream) {
  g_err.clear();
  Prob o;
  TRY(to_prob(p, o, false));
  if (!std::isfinite(dense_above) || dense_above < 0.f)
    return fail(DSV_ERR_INVALID_ARGUMENT, "dense_above must be finite and >= 0");
  if (block_counts) TRY(check_ptr(block_counts, "block_counts", 4));
  TRY(check_ptr(density, "density", 4));
  if (dense) TRY(check_ptr(dense, "dense", 4));
  const double cells = (double)o.nqb() * (double)o.nkb();
  const long long limit = (long long)std::floor((double)dense_above * cells);
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY_HIP(dsv::launch_head_density(block_counts, density, dense, o.nqb(), o.k, o.nkb(), limit, o.bh(), st),
          "head_density_kernel");
  return DSV_OK;
}

dsv_status dsv_block_recall(const dsv_problem* p, const float* lse_selected, const float* lse_all, float* recall,
                            void* stream) {
  g_err.clear();
  Prob o;
  TRY(to_prob(p, o, false));
  TRY(check_ptr(lse_selected, "lse_selected", 4));
  TRY(check_ptr(lse_all, "lse_all", 4));
  TRY(check_ptr(recall, "recall", 4));
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY_HIP(dsv::launch_block_recall(lse_selected, lse_all, recall, o.bh() * o.nqb(), o.bq, st), "block_recall_kernel");
  return DSV_OK;
}

size_t dsv_pack_kv_workspace_size(const dsv_problem* p) {
  Prob o;
  if (to_prob(p, o, false) != DSV_OK) return 0;
  return 2 * align_up((size_t)o.bh() * o.nkb() * 4);
}

namespace {
// the checks shared by dsv_pack_kv and dsv_pack_kv_noalloc (everything but the scratch)
dsv_status check_pack(const dsv_problem* p, Prob& o, const void* k, const void* v, const int32_t* block_idx,
                      const int32_t* block_counts, int32_t qb_begin, int32_t qb_end, const void* k_packed,
                      const void* v_packed, const int32_t* packed_blocks, const int32_t* packed_counts,
                      const int32_t* packed_idx) {
  TRY(to_prob(p, o, false));
  if (qb_begin < 0 || qb_end > o.nqb() || qb_begin > qb_end)
    return fail(DSV_ERR_INVALID_ARGUMENT, "need 0 <= qb_begin <= qb_end <= N/Bq");
  const void* ptrs[] = {k, v, k_packed, v_packed};
  const char* names[] = {"k", "v", "k_packed", "v_packed"};
  for (int i = 0; i < 4; ++i) TRY(check_ptr(ptrs[i], names[i]));
  TRY(check_ptr(block_idx, "block_idx", 4));
  if (block_counts) TRY(check_ptr(block_counts, "block_counts", 4));
  TRY(check_ptr(packed_blocks, "packed_blocks", 4));
  TRY(check_ptr(packed_counts, "packed_counts", 4));
  if (qb_end > qb_begin) TRY(check_ptr(packed_idx, "packed_idx", 4));
  if (o.bk != 64) return fail(DSV_ERR_UNSUPPORTED, "packing needs Bk = 64");
  return DSV_OK;
}
}  // namespace

dsv_status dsv_pack_kv(const dsv_problem* p, const void* k, const void* v, const int32_t* block_idx,
                       const int32_t* block_counts, int32_t qb_begin, int32_t qb_end, void* k_packed, void* v_packed,
                       int32_t* packed_blocks, int32_t* packed_counts, int32_t* packed_idx, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_err.clear();
  Prob o;
  TRY(check_pack(p, o, k, v, block_idx, block_counts, qb_begin, qb_end, k_packed, v_packed, packed_blocks,
                 packed_counts, packed_idx));
  TRY(check_ptr(workspace, "workspace", kWsAlign));
  const size_t half = align_up((size_t)o.bh() * o.nkb() * 4);
  if (workspace_bytes < 2 * half)
    return fail(DSV_ERR_WORKSPACE_TOO_SMALL, "pack workspace needs " + std::to_string(2 * half) + " bytes");
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY_HIP(dsv::launch_pack_kv(k, v, block_idx, block_counts, k_packed, v_packed, packed_blocks, packed_counts,
                              packed_idx, at<int32_t>(workspace, 0), at<int32_t>(workspace, half), o.bh(), o.n,
                              (int)(o.d * o.esize()), o.nqb(), o.nkb(), o.k, qb_begin, qb_end, st),
          "pack_kernels");
  return DSV_OK;
}

dsv_status dsv_pack_kv_noalloc(const dsv_problem* p, const void* k, const void* v, const int32_t* block_idx,
                               const int32_t* block_counts, int32_t qb_begin, int32_t qb_end, void* k_packed,
                               void* v_packed, int32_t* packed_blocks, int32_t* packed_counts, int32_t* packed_idx,
                               void* stream) {
  g_err.clear();
  Prob o;
  TRY(to_prob(p, o, false));
  const size_t need = (size_t)o.bh() * o.nkb();
  if (need > dsv::kPackScratchEntries)
    return fail(DSV_ERR_UNSUPPORTED, "B*H*N/Bk = " + std::to_string(need) + " exceeds the allocation-free limit of " +
                                         std::to_string(dsv::kPackScratchEntries) + " (use dsv_pack_kv)");
  TRY(check_pack(p, o, k, v, block_idx, block_counts, qb_begin, qb_end, k_packed, v_packed, packed_blocks,
                 packed_counts, packed_idx));
  int32_t *flags = nullptr, *pos = nullptr;
  TRY(hip_status(dsv::pack_scratch(&flags, &pos), "pack scratch lookup"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY_HIP(dsv::launch_pack_kv(k, v, block_idx, block_counts, k_packed, v_packed, packed_blocks, packed_counts,
                              packed_idx, flags, pos, o.bh(), o.n, (int)(o.d * o.esize()), o.nqb(), o.nkb(), o.k,
                              qb_begin, qb_end, st),
          "pack_kernels");
  return DSV_OK;
}

size_t dsv_sparse_attn_fwd_workspace_size(const dsv_problem* p) {
  Prob o;
  if (to_prob(p, o, false) != DSV_OK) return 0;
  return fwd_ws_bytes(o);
}

dsv_status dsv_sparse_attn_fwd(const dsv_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, const int32_t* block_counts, void* o_ptr, float* lse,
                               void* o_lo, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  Prob o;
  TRY(to_prob(p, o, false));
  TRY(check_bf16_attn(o));
  TRY(check_f32_attn(o));
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  TRY(check_ptr(block_idx, "block_idx", 4));
  if (block_counts) TRY(check_ptr(block_counts, "block_counts", 4));
  TRY(check_ptr(o_ptr, "o"));
  TRY(check_ptr(lse, "lse"));
  TRY(check_residual(o, o_lo));
  const size_t need = o_lo ? fwd_ws_bytes(o) : 0;
  if (need) {
    TRY(check_ptr(workspace, "workspace", kWsAlign));
    if (workspace_bytes < need)
      return fail(DSV_ERR_WORKSPACE_TOO_SMALL, "forward workspace needs " + std::to_string(need) + " bytes");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY(check_lists(o, block_idx, block_counts, st));
  if (o.dtype == DSV_BF16) {
    TRY_HIP(dsv::launch_attn_fwd_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                      static_cast<const uint16_t*>(v), block_idx, block_counts,
                                      static_cast<uint16_t*>(o_ptr), lse, static_cast<uint16_t*>(o_lo), workspace,
                                      o.bh(), o.n, o.d, o.bq, o.k, o.sm, st),
            "attn_fwd_kernel");
  } else {
    TRY_HIP(dsv::launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                     static_cast<const float*>(v), block_idx, block_counts,
                                     static_cast<float*>(o_ptr), lse, o.bh(),
                                     o.n, o.d, o.bq, o.bk, o.k, o.sm, st), "attn_fwd_kernel");
  }
  return DSV_OK;
}

size_t dsv_sparse_attn_bwd_workspace_size(const dsv_problem* p) {
  Prob o;
  if (to_prob(p, o, false) != DSV_OK) return 0;
  return bwd_ws(o).total;
}

dsv_status dsv_sparse_attn_bwd(const dsv_problem* p, const void* q, const void* k, const void* v, const void* o_ptr,
                               const void* o_lo, const void* dout, const float* lse, const int32_t* block_idx,
                               const int32_t* block_counts, void* dq, void* dk,
                               void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  Prob o;
  TRY(to_prob(p, o, false));
  TRY(check_bf16_attn(o));
  TRY(check_f32_attn(o));
  const void* ptrs[] = {q, k, v, o_ptr, dout, lse, dq, dk, dv};
  const char* names[] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"};
  for (int i = 0; i < 9; ++i) TRY(check_ptr(ptrs[i], names[i]));
  TRY(check_ptr(block_idx, "block_idx", 4));
  if (block_counts) TRY(check_ptr(block_counts, "block_counts", 4));
  // the dQ kernel's fp16 products scale S by up to 2^+-80 and fold the inverse into sm_scale
  if (o.dtype == DSV_BF16 && !(o.sm >= 0x1p-40f && o.sm <= 0x1p40f))
    return fail(DSV_ERR_UNSUPPORTED, "the bf16 backward needs sm_scale in [2^-40, 2^40]");
  TRY(check_residual(o, o_lo));
  TRY(check_ptr(workspace, "workspace", kWsAlign));
  const BwdWs w = bwd_ws(o);
  if (workspace_bytes < w.total)
    return fail(DSV_ERR_WORKSPACE_TOO_SMALL, "backward workspace needs " + std::to_string(w.total) + " bytes");
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY(check_lists(o, block_idx, block_counts, st));
  int32_t* col_ptr = at<int32_t>(workspace, w.col_ptr);
  int32_t* rows = at<int32_t>(workspace, w.rows);
  int32_t* order = o.dtype == DSV_BF16 ? at<int32_t>(workspace, w.order) : nullptr;
  TRY_HIP(dsv::launch_csc(block_idx, block_counts, at<uint32_t>(workspace, w.bitmap), at<int32_t>(workspace, w.counts),
                          col_ptr, rows, order, o.bh(), o.nqb(), o.nkb(), o.k, st), "csc_kernels");
  float* dvec = at<float>(workspace, w.dvec);
  if (o.dtype == DSV_BF16) {
    const uint16_t* q16 = static_cast<const uint16_t*>(q);
    const uint16_t* k16 = static_cast<const uint16_t*>(k);
    const uint16_t* v16 = static_cast<const uint16_t*>(v);
    const uint16_t* do16 = static_cast<const uint16_t*>(dout);
    float* lse2 = at<float>(workspace, w.lse2);
    void* f16 = at<void>(workspace, w.f16);
    float* dvec_s = at<float>(workspace, w.dvec_s);
    TRY_HIP(dsv::launch_bwd_prep_bf16(q16, k16, v16, do16, f16, o.bh(), o.n, o.d, st), "bwd_prep_kernels");
    TRY_HIP(dsv::launch_bwd_pre_bf16(static_cast<const uint16_t*>(o_ptr), static_cast<const uint16_t*>(o_lo), do16,
                                     lse, dvec, lse2, dvec_s, f16, o.bh(), o.n, o.d, st), "bwd_pre_kernel");
    TRY_HIP(dsv::launch_bwd_dkdv_bf16(f16, v16, do16, lse2, dvec_s, col_ptr, rows, order, static_cast<uint16_t*>(dk),
                                      static_cast<uint16_t*>(dv), o.bh(), o.n, o.d, o.bq, o.k, o.sm, st),
            "attn_bwd_dkdv_kernel");
    TRY_HIP(dsv::launch_bwd_dq_bf16(q16, v16, do16, lse2, dvec, block_idx, block_counts, static_cast<uint16_t*>(dq),
                                    f16, o.bh(), o.n, o.d, o.bq, o.k, o.sm, st),
            "attn_bwd_dq_kernel");
  } else {
    TRY_HIP(dsv::launch_bwd_pre_f32(static_cast<const float*>(o_ptr), static_cast<const float*>(dout), dvec,
                                    o.bh() * o.n, o.d, st), "bwd_pre_kernel");
    TRY_HIP(dsv::launch_bwd_f32(static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                                static_cast<const float*>(dout), lse, dvec, block_idx, block_counts, col_ptr, rows,
                                static_cast<float*>(dq), static_cast<float*>(dk), static_cast<float*>(dv), o.bh(), o.n,
                                o.d, o.bq, o.bk, o.k, o.sm, st), "attn_bwd_f32_kernels");
  }
  return DSV_OK;
}

}  // extern "C"
