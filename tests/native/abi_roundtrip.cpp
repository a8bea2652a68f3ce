// A native caller of the C ABI: the whole hot path (predict -> top-k -> sparse forward ->
// sparse backward) through include/dsv.h with plain hipMalloc'd buffers, no Python and no
// torch.  The GPU test that runs it compares its outputs with the Python binding's, bit for bit.
//
//   abi_roundtrip IN OUT B H N d r Bq k
// IN holds, as raw little-endian bf16 bit patterns: q, k, v, dout ([B,H,N,d] each), then wq, wk
// ([H,d,r] each).  OUT receives: block scores (float32 [B,H,N/Bq,N/64]), block lists (int32
// [B,H,N/Bq,k]), o (bf16), lse (float32 [B,H,N]), dq, dk, dv (bf16).
// Exit status: 0 ok, 1 usage or file error, 2 a library call failed, 3 a HIP call failed.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/dsv.h"

#define CHECK_DSV(call)                                                                                  \
  do {                                                                                                   \
    const dsv_status st_ = (call);                                                                       \
    if (st_ != DSV_OK) {                                                                                 \
      std::fprintf(stderr, "%s failed: %s (%s)\n", #call, dsv_status_string(st_), dsv_last_error());     \
      return 2;                                                                                          \
    }                                                                                                    \
  } while (0)
#define CHECK_HIP(call)                                                                                  \
  do {                                                                                                   \
    const hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess) {                                                                              \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));                             \
      return 3;                                                                                          \
    }                                                                                                    \
  } while (0)

namespace {

struct Buf {
  void* p = nullptr;
  ~Buf() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

int main(int argc, char** argv) {
  if (argc != 10) {
    std::fprintf(stderr, "usage: %s IN OUT B H N d r Bq k\n", argv[0]);
    return 1;
  }
  dsv_problem p{};
  p.batch = std::atoi(argv[3]);
  p.heads = std::atoi(argv[4]);
  p.seq_len = std::atoi(argv[5]);
  p.head_dim = std::atoi(argv[6]);
  p.rank = std::atoi(argv[7]);
  p.q_block = std::atoi(argv[8]);
  p.topk = std::atoi(argv[9]);
  p.kv_block = 64;
  p.dtype = DSV_BF16;
  p.sm_scale = 0.f;    // 1/sqrt(d)
  p.pred_scale = 0.f;  // 1/sqrt(d)
  if (p.batch < 1 || p.heads < 1 || p.seq_len < 1 || p.head_dim < 1 || p.rank < 1 || p.q_block < 1 || p.topk < 1) {
    std::fprintf(stderr, "bad sizes\n");
    return 1;
  }
  const size_t bh = (size_t)p.batch * p.heads, n = (size_t)p.seq_len, d = (size_t)p.head_dim;
  const size_t nqb = n / p.q_block, nkb = n / p.kv_block;
  const size_t act = bh * n * d, wts = (size_t)p.heads * d * p.rank;

  std::vector<uint16_t> host(4 * act + 2 * wts);
  FILE* f = std::fopen(argv[1], "rb");
  if (!f || std::fread(host.data(), 2, host.size(), f) != host.size()) {
    std::fprintf(stderr, "cannot read %s\n", argv[1]);
    if (f) std::fclose(f);
    return 1;
  }
  std::fclose(f);

  // device buffers
  Buf q, k, v, dout, wq, wk, scores, idx, o, o_lo, lse, dq, dk, dv, wsp, wsf, wsb;
  CHECK_HIP(hipMalloc(&q.p, act * 2));
  CHECK_HIP(hipMalloc(&k.p, act * 2));
  CHECK_HIP(hipMalloc(&v.p, act * 2));
  CHECK_HIP(hipMalloc(&dout.p, act * 2));
  CHECK_HIP(hipMalloc(&wq.p, wts * 2));
  CHECK_HIP(hipMalloc(&wk.p, wts * 2));
  CHECK_HIP(hipMalloc(&scores.p, bh * nqb * nkb * 4));
  CHECK_HIP(hipMalloc(&idx.p, bh * nqb * p.topk * 4));
  CHECK_HIP(hipMalloc(&o.p, act * 2));
  CHECK_HIP(hipMalloc(&o_lo.p, act * 2));
  CHECK_HIP(hipMalloc(&lse.p, bh * n * 4));
  CHECK_HIP(hipMalloc(&dq.p, act * 2));
  CHECK_HIP(hipMalloc(&dk.p, act * 2));
  CHECK_HIP(hipMalloc(&dv.p, act * 2));
  const size_t np = dsv_predict_workspace_size(&p), nf = dsv_sparse_attn_fwd_workspace_size(&p),
               nb = dsv_sparse_attn_bwd_workspace_size(&p);
  if (!np || !nf || !nb) {
    std::fprintf(stderr, "unsupported problem: %s\n", dsv_last_error());
    return 2;
  }
  CHECK_HIP(hipMalloc(&wsp.p, np));
  CHECK_HIP(hipMalloc(&wsf.p, nf));
  CHECK_HIP(hipMalloc(&wsb.p, nb));
  const uint16_t* h = host.data();
  CHECK_HIP(hipMemcpy(q.p, h, act * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k.p, h + act, act * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v.p, h + 2 * act, act * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dout.p, h + 3 * act, act * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(wq.p, h + 4 * act, wts * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(wk.p, h + 4 * act + wts, wts * 2, hipMemcpyHostToDevice));

  // the hot path, all on the null stream
  CHECK_DSV(dsv_predict(&p, q.p, k.p, wq.p, wk.p, wsp.p, np, static_cast<float*>(scores.p), nullptr));
  CHECK_DSV(dsv_select_topk(&p, static_cast<const float*>(scores.p), static_cast<int32_t*>(idx.p), nullptr));
  CHECK_DSV(dsv_sparse_attn_fwd(&p, q.p, k.p, v.p, static_cast<const int32_t*>(idx.p), nullptr, o.p,
                                static_cast<float*>(lse.p), o_lo.p, wsf.p, nf, nullptr));
  CHECK_DSV(dsv_sparse_attn_bwd(&p, q.p, k.p, v.p, o.p, o_lo.p, dout.p, static_cast<const float*>(lse.p),
                                static_cast<const int32_t*>(idx.p), nullptr, dq.p, dk.p, dv.p, wsb.p, nb, nullptr));
  CHECK_HIP(hipDeviceSynchronize());

  // results back to the host, in the order documented above
  struct Out {
    const Buf* b;
    size_t bytes;
  } outs[] = {{&scores, bh * nqb * nkb * 4}, {&idx, bh * nqb * p.topk * 4}, {&o, act * 2}, {&lse, bh * n * 4},
              {&dq, act * 2},                {&dk, act * 2},                {&dv, act * 2}};
  FILE* g = std::fopen(argv[2], "wb");
  if (!g) {
    std::fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  std::vector<char> tmp;
  for (const Out& x : outs) {
    tmp.resize(x.bytes);
    CHECK_HIP(hipMemcpy(tmp.data(), x.b->p, x.bytes, hipMemcpyDeviceToHost));
    if (std::fwrite(tmp.data(), 1, x.bytes, g) != x.bytes) {
      std::fclose(g);
      return 1;
    }
  }
  std::fclose(g);
  std::printf("abi_roundtrip: ok (library version %d)\n", dsv_version());
  return 0;
}
