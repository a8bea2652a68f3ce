"""GPU parity over a seeded sweep of shapes: each case draws one compiled bf16 instance (d, Bq, r),
a sequence length that is a multiple of 256 up to 2048, a batch of one or two and one to three
heads, a k between 1 and every block (every block in three cases), and in half the cases ragged
lists (per-query-block counts, some of them 0).  The whole path runs through the C ABI --
predict, top-k, the training forward and the backward -- and is compared with the oracle: scores
fed the GPU's own projections (rtol 2e-4, atol 2e-5), indices under the gap rule, O, LSE and
gradients on the GPU's lists.  A second sweep does the same for the fp32 path over its wider
shape range (any d <= 128, r <= 64, Bk | Bq | N)."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from oracle import dsv_oracle as O
from tests.gpu_helpers import (FWD_BF16_MAXABS, FWD_BF16_RELL2, GRAD_BF16_MAXABS, check_indices, log, rel_l2,
                               to_dev, to_f64)
from workloads.generator import bf16_bits_from_f32, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsv.load_library()
    yield
    torch.cuda.synchronize()


def _case(seed):
    rng = np.random.default_rng(7000 + seed)
    d = int(rng.choice([64, 128]))
    bq = int(rng.choice([64, 128]))
    r = int(rng.choice([16, 32]))
    n = 256 * int(rng.integers(1, 9))
    b, h = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    nkb = n // 64
    k = nkb if seed % 8 == 4 else int(rng.integers(1, nkb + 1))  # every block, now and then
    return rng, d, bq, r, n, b, h, k, seed % 2 == 1


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_match_the_oracle(seed):
    rng, d, bq, r, n, b, h, k, ragged = _case(seed)
    log(f"[parity] sweep seed={seed}: B={b} H={h} N={n} d={d} r={r} Bq={bq} k={k} ragged={ragged}")
    nqb, bk = n // bq, 64

    def bf(shape, scale=1.0):
        return bf16_bits_from_f32((rng.standard_normal(shape) * scale).astype(np.float32))

    inp = {"q": bf((b, h, n, d)), "k": bf((b, h, n, d)), "v": bf((b, h, n, d)), "do": bf((b, h, n, d)),
           "wq": bf((h, d, r), 1 / np.sqrt(d)), "wk": bf((h, d, r), 1 / np.sqrt(d))}
    t = {nm: to_dev(a) for nm, a in inp.items()}
    kw = dict(q_block=bq, kv_block=bk)
    scores, qlr, klr = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], return_projections=True, **kw)
    idx = dsv.select_topk(scores, k, **kw)
    cnt = None
    if ragged:
        cnt = torch.from_numpy(rng.integers(0, k + 1, size=(b, h, nqb)).astype(np.int32)).cuda()
    o, lse, o_lo = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, residual=True, block_counts=cnt, **kw)
    grads = dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, idx, o_lo=o_lo, block_counts=cnt, **kw)
    torch.cuda.synchronize()

    sg, ql, kl, gi = to_f64(scores), to_f64(qlr), to_f64(klr), idx.cpu().numpy()
    for bi in range(b):
        for hi in range(h):
            ref = O.block_scores_head(ql[bi, hi], kl[bi, hi], bq, bk, O.LN2)
            np.testing.assert_allclose(sg[bi, hi], ref, rtol=2e-4, atol=2e-5, err_msg=f"scores b{bi} h{hi}")
            check_indices(gi[bi, hi], ref, k)
    lists = gi.copy()
    if ragged:
        c = cnt.cpu().numpy()
        lists[np.arange(k) >= c[..., None]] = -1  # entries past the count select nothing
    x = {nm: widen(a) for nm, a in inp.items()}
    sc = 1.0 / np.sqrt(d)
    o_o, lse_o = O.sparse_attn_fwd(x["q"], x["k"], x["v"], lists, bq, bk, sc)
    og, lg = to_f64(o), to_f64(lse)
    assert np.abs(og - o_o).max() <= FWD_BF16_MAXABS and rel_l2(og, o_o) <= FWD_BF16_RELL2
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lg), fin)  # empty lists: LSE = -inf
    assert np.abs(lg[fin] - lse_o[fin]).max() <= 1e-3
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], lists, bq, bk, sc)
    for nm, got, ref in zip(("dq", "dk", "dv"), grads, g_o):
        err = np.abs(to_f64(got) - ref).max()
        assert err <= GRAD_BF16_MAXABS, (nm, err)
    log(f"[parity] sweep seed={seed}: scores, indices, O, LSE and gradients match")


def _case_f32(seed):
    rng = np.random.default_rng(9000 + seed)
    d = int(rng.choice([16, 32, 48, 64, 96, 128]))
    r = int(rng.choice([8, 16, 32, 64]))
    bk = int(rng.choice([16, 32, 64]))
    bq = bk * int(rng.choice([1, 2, 4]))
    n = bq * int(rng.integers(2, max(3, 1024 // bq) + 1))
    b, h = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    nkb = n // bk
    k = nkb if seed % 6 == 3 else int(rng.integers(1, nkb + 1))
    return rng, d, bq, bk, r, n, b, h, k, seed % 2 == 1


@pytest.mark.parametrize("seed", range(12))
def test_random_f32_shapes_match_the_oracle(seed):
    # The fp32 path takes any d <= 128, r <= 64 and any Bq, Bk with Bk | Bq | N: fp32 bounds of
    # 1e-5 on O and the LSE, 1e-4 on the gradients, the oracle fed the GPU's projections.
    rng, d, bq, bk, r, n, b, h, k, ragged = _case_f32(seed)
    log(f"[parity] f32 sweep seed={seed}: B={b} H={h} N={n} d={d} r={r} Bq={bq} Bk={bk} k={k} ragged={ragged}")
    nqb = n // bq
    inp = {nm: rng.standard_normal(shape).astype(np.float32) for nm, shape in
           (("q", (b, h, n, d)), ("k", (b, h, n, d)), ("v", (b, h, n, d)), ("do", (b, h, n, d)))}
    inp["wq"] = (rng.standard_normal((h, d, r)) / np.sqrt(d)).astype(np.float32)
    inp["wk"] = (rng.standard_normal((h, d, r)) / np.sqrt(d)).astype(np.float32)
    t = {nm: to_dev(a) for nm, a in inp.items()}
    kw = dict(q_block=bq, kv_block=bk)
    scores, qlr, klr = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], return_projections=True, **kw)
    idx = dsv.select_topk(scores, k, **kw)
    cnt = None
    if ragged:
        cnt = torch.from_numpy(rng.integers(0, k + 1, size=(b, h, nqb)).astype(np.int32)).cuda()
    o, lse = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, block_counts=cnt, **kw)
    grads = dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, idx, block_counts=cnt, **kw)
    torch.cuda.synchronize()

    sg, ql, kl, gi = to_f64(scores), to_f64(qlr), to_f64(klr), idx.cpu().numpy()
    for bi in range(b):
        for hi in range(h):
            ref = O.block_scores_head(ql[bi, hi], kl[bi, hi], bq, bk, O.LN2)
            np.testing.assert_allclose(sg[bi, hi], ref, rtol=1e-4, atol=1e-5, err_msg=f"scores b{bi} h{hi}")
            check_indices(gi[bi, hi], ref, k)
    lists = gi.copy()
    if ragged:
        c = cnt.cpu().numpy()
        lists[np.arange(k) >= c[..., None]] = -1
    x = {nm: a.astype(np.float64) for nm, a in inp.items()}
    sc = 1.0 / np.sqrt(d)
    o_o, lse_o = O.sparse_attn_fwd(x["q"], x["k"], x["v"], lists, bq, bk, sc)
    assert np.abs(to_f64(o) - o_o).max() <= 1e-5
    lg, fin = to_f64(lse), np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lg), fin) and np.abs(lg[fin] - lse_o[fin]).max() <= 1e-5
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], lists, bq, bk, sc)
    for nm, got, ref in zip(("dq", "dk", "dv"), grads, g_o):
        err = np.abs(to_f64(got) - ref).max()
        assert err <= 1e-4, (nm, err)
    log(f"[parity] f32 sweep seed={seed}: scores, indices, O, LSE and gradients match")
