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
from tests.gpu_helpers import log, to_dev, to_f64
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
