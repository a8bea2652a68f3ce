"""GPU parity of the representative-row predictor: each query block is scored by the predicted
softmax mass of one of its rows ([de] §2.B, query grouping).  The oracle is fed the GPU's own
projections, as for the block-score predictor; scores match to rtol 2e-4 (atol 1e-6, rows sum to
1), and top-k on them matches the oracle's wherever the oracle's k-th/(k+1)-th gap exceeds 1e-5
(five times the score error bound at the scores' ~1e-2 scale)."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from oracle import dsv_oracle as O
from tests.gpu_helpers import check_indices, log, to_dev, to_f64
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu
REP_GAP = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsv.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,rep", [("C2", 0), ("C2", 63), ("C3", 17), ("C1", 5)])
def test_representative_scores_and_selection(name, rep):
    cfg = get_config(name)
    heads = list(range(min(cfg.heads, 3)))
    cfg = cfg.with_(heads=len(heads))
    inp = make_inputs(cfg, with_grad=False)
    t = {k: to_dev(v) for k, v in inp.items() if k in ("q", "k", "wq", "wk")}
    scores, qlr, klr = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], q_block=cfg.q_block, kv_block=cfg.kv_block,
                                   rep_row=rep, return_projections=True)
    k = min(cfg.topk, cfg.nkb)
    idx = dsv.select_topk(scores, k, q_block=cfg.q_block, kv_block=cfg.kv_block)
    torch.cuda.synchronize()
    sg, ig = to_f64(scores), idx.cpu().numpy()
    covered = []
    for h in range(cfg.heads):
        ref = O.representative_scores_head(to_f64(qlr)[0, h], to_f64(klr)[0, h], cfg.q_block, cfg.kv_block, O.LN2,
                                           rep=rep)  # qlr: the scaled query operand Q~
        np.testing.assert_allclose(sg[0, h], ref, rtol=2e-4, atol=1e-6)
        np.testing.assert_allclose(sg[0, h].sum(-1), 1.0, rtol=1e-4)
        ref_idx, gap = O.select_topk(ref, k), O.topk_gap(ref, k)
        exact = gap > REP_GAP
        assert np.array_equal(ig[0, h][exact], ref_idx[exact])
        covered.append(exact.mean())
    log(f"[parity] representative {name} rep={rep}: rows under the exact index rule {np.mean(covered):.3f}")


# ------------------------------------------------------------------ fused predictor + top-k


def _fused_vs_oracle(cfg, inp, rep, heads_checked):
    t = {k: to_dev(v) for k, v in inp.items() if k in ("q", "k", "wq", "wk")}
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block)
    idx, qlr, klr = dsv.predict_select_representative(t["q"], t["k"], t["wq"], t["wk"], cfg.topk, rep,
                                                      return_projections=True, **kw)
    # the unfused pair on the same inputs: dsv_predict_representative then dsv_select_topk
    sc = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], rep_row=rep, **kw)
    idx_u = dsv.select_topk(sc, cfg.topk, **kw)
    torch.cuda.synchronize()
    ig, iu, ql, kl = idx.cpu().numpy(), idx_u.cpu().numpy(), to_f64(qlr), to_f64(klr)
    cov = []
    for h in heads_checked:
        ref = O.representative_scores_head(ql[0, h], kl[0, h], cfg.q_block, cfg.kv_block, O.LN2, rep=rep)
        cov.append(check_indices(ig[0, h], ref, cfg.topk, gap_rule=REP_GAP))
        exact = O.topk_gap(ref, cfg.topk) > REP_GAP
        assert np.array_equal(ig[0, h][exact], iu[0, h][exact])  # the fused and unfused paths agree there
    return float(np.mean(cov))


@pytest.mark.parametrize("name,rep", [("C2", 0), ("C2", 63), ("C3", 17), ("C5", 64), ("C1", 5)])
def test_fused_representative_selection(name, rep):
    # dsv_predict_select_representative: the top-k of each query block's representative row straight
    # from the projections (the bf16 kernel ranks blocks by their unnormalised mass inside the
    # sweep), against the oracle's representative scores and top-k: bit-exact wherever the oracle's
    # k-th/(k+1)-th gap exceeds 1e-5, valid near-tie choices elsewhere.  C5: 2 heads at full size
    # (2048 KV blocks, 1024 query blocks).
    cfg = get_config(name)
    cfg = cfg.with_(heads=2 if name == "C5" else min(cfg.heads, 3))
    log(f"[parity] fused representative {name} rep={rep} N={cfg.seq_len} k={cfg.topk}")
    inp = make_inputs(cfg, with_grad=False, workers=8)
    cov = _fused_vs_oracle(cfg, inp, rep, range(cfg.heads))
    log(f"[parity] fused representative {name} rep={rep}: rows under the exact index rule {cov:.3f}")


@pytest.mark.parametrize("n,heads,topk", [(256, 5, 2), (4352, 3, 7), (262144, 1, 410)])
def test_fused_representative_edge_sizes(n, heads, topk):
    # N = 256: 4 KV blocks, one per wave; N = 4352: 68 KV blocks (17 per wave, odd), 34 query blocks
    # (a work item with rows past the last query block); N = 262144: 4096 KV blocks (64 keys per lane
    # in the selection), 2048 query blocks.  G1-style inputs at d = 128, r = 32, Bq = 128.
    cfg = get_config("C5").with_(latent=(1, 1, n), heads=heads, topk=topk)
    log(f"[parity] fused representative edge N={n} heads={heads} k={topk}")
    inp = make_inputs(cfg, with_grad=False, workers=8)
    cov = _fused_vs_oracle(cfg, inp, 3, range(heads))
    log(f"[parity] fused representative N={n}: rows under the exact index rule {cov:.3f}")


@pytest.mark.parametrize("case", ["overflow", "tiny"])
def test_fused_representative_extreme_logits(case):
    # Logits far beyond fp32's exponent range (2^+-138 per key): the block masses overflow or
    # vanish, the item is swept again with in-block log-sum-exp keys, which stay exact, so block 5
    # -- the only block with the largest logits -- leads every selection.
    n, d, r, bq, bk, k = 1024, 64, 16, 64, 64, 3
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, 1, n, d)).astype(np.float32) * 0.1
    kk = rng.standard_normal((1, 1, n, d)).astype(np.float32) * 0.1
    q[..., :r] = 1.0
    if case == "overflow":
        kk[0, 0, :, :r] = 24.0 + np.abs(kk[0, 0, :, :r]) * 20
        kk[0, 0, 5 * 64:6 * 64, :r] = 48.0
    else:
        kk[0, 0, :, :r] = -48.0 - np.abs(kk[0, 0, :, :r]) * 200
        kk[0, 0, 5 * 64:6 * 64, :r] = -48.0
    w = np.zeros((1, d, r), np.float32)
    w[0, :r, :r] = np.eye(r)
    from workloads.generator import bf16_bits_from_f32
    t = {nm: to_dev(bf16_bits_from_f32(a)) for nm, a in (("q", q), ("k", kk), ("w", w))}
    idx, qlr, klr = dsv.predict_select_representative(t["q"], t["k"], t["w"], t["w"], k, 7, q_block=bq, kv_block=bk,
                                                      return_projections=True)
    torch.cuda.synchronize()
    ref = O.representative_scores_head(to_f64(qlr)[0, 0], to_f64(klr)[0, 0], bq, bk, O.LN2, rep=7)
    ig = idx.cpu().numpy()[0, 0]
    check_indices(ig, ref, k, gap_rule=REP_GAP)
    assert np.all(np.any(ig == 5, axis=1))


@pytest.mark.parametrize("seed", range(8))
def test_representative_paths_over_random_shapes(seed):
    # Seeded shapes over the bf16 instances: d, Bq and r drawn from the compiled ones, N a multiple
    # of 256 up to 4096, one to three heads, a random representative row and k.  Both paths --
    # scores then top-k, and the fused selection -- against the oracle on the GPU's projections.
    rng = np.random.default_rng(5100 + seed)
    d, bq, r = int(rng.choice([64, 128])), int(rng.choice([64, 128])), int(rng.choice([16, 32]))
    n, heads = 256 * int(rng.integers(1, 17)), int(rng.integers(1, 4))
    nkb = n // 64
    k, rep = int(rng.integers(1, nkb + 1)), int(rng.integers(0, bq))
    log(f"[parity] representative sweep seed={seed}: H={heads} N={n} d={d} r={r} Bq={bq} k={k} rep={rep}")
    from workloads.generator import bf16_bits_from_f32
    bf = lambda shape, s=1.0: bf16_bits_from_f32((rng.standard_normal(shape) * s).astype(np.float32))  # noqa: E731
    t = {"q": to_dev(bf((1, heads, n, d))), "k": to_dev(bf((1, heads, n, d))),
         "wq": to_dev(bf((heads, d, r), 1 / np.sqrt(d))), "wk": to_dev(bf((heads, d, r), 1 / np.sqrt(d)))}
    kw = dict(q_block=bq, kv_block=64)
    sc, qlr, klr = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], rep_row=rep, return_projections=True, **kw)
    iu = dsv.select_topk(sc, k, **kw)
    ig = dsv.predict_select_representative(t["q"], t["k"], t["wq"], t["wk"], k, rep, **kw)
    torch.cuda.synchronize()
    sg, ql, kl = to_f64(sc), to_f64(qlr), to_f64(klr)
    iu, ig = iu.cpu().numpy(), ig.cpu().numpy()
    for h in range(heads):
        ref = O.representative_scores_head(ql[0, h], kl[0, h], bq, 64, O.LN2, rep=rep)
        np.testing.assert_allclose(sg[0, h], ref, rtol=2e-4, atol=1e-6, err_msg=f"head {h}")
        check_indices(iu[0, h], ref, k, gap_rule=REP_GAP)
        check_indices(ig[0, h], ref, k, gap_rule=REP_GAP)
        exact = O.topk_gap(ref, k) > REP_GAP
        assert np.array_equal(ig[0, h][exact], iu[0, h][exact])
