"""GPU parity of the selection profiler's recall: the true attention mass a selection captures,
per query block ([de] §2.A).  The GPU forms it from two forward lse (the selection's, and every
block's); the oracle from the dense fp64 softmax over all keys, summed over the selected keys --
an independent route to the same number.  Both lse are float32 log-sum-exps of products
accumulated in float32 (exact for bf16 inputs), each within a few units in the last place of a
value below ~20 (ulp 2e-6) after the blocked float32 sums; recall = exp of their difference is at
most 1, so its absolute error is bounded by that difference's: held to 1e-5."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from oracle import dsv_oracle as O
from tests.gpu_helpers import log, to_dev
from workloads import get_config, make_inputs
from workloads.generator import widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsv.load_library()
    yield
    torch.cuda.synchronize()


def _recall_case(cfg, tol, mass_tau=None):
    inp = make_inputs(cfg, with_grad=False)
    x = {k: widen(v) for k, v in inp.items() if k in ("q", "k")}
    t = {k: to_dev(v) for k, v in inp.items() if k in ("q", "k", "v", "wq", "wk")}
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block)
    scores = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], **kw)
    if mass_tau is None:
        idx, cnt = dsv.select_topk(scores, min(cfg.topk, cfg.nkb), **kw), None
    else:
        idx, cnt = dsv.select_mass(scores, mass_tau, min(cfg.topk, cfg.nkb), **kw)
    lse_sel = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, block_counts=cnt, **kw)[1]
    b, h = t["q"].shape[:2]
    idx_all = torch.arange(cfg.nkb, dtype=torch.int32, device=idx.device).repeat(b, h, cfg.nqb, 1).contiguous()
    lse_all = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx_all, **kw)[1]
    rec = dsv.block_recall(lse_sel, lse_all, q_block=cfg.q_block)
    torch.cuda.synchronize()
    lists = idx.cpu().numpy().copy()
    if cnt is not None:
        lists[np.arange(lists.shape[-1]) >= cnt.cpu().numpy()[..., None]] = -1
    ref = O.block_recall(x["q"], x["k"], lists, cfg.q_block, cfg.kv_block, 1.0 / np.sqrt(cfg.head_dim))
    got = rec.double().cpu().numpy()
    err = np.abs(got - ref).max()
    log(f"[parity] recall {cfg.name} tau={mass_tau}: mean {ref.mean():.4f} min {ref.min():.4f}, max-abs {err:.2e}")
    assert got.shape == ref.shape and np.all((got >= 0) & (got <= 1 + tol))
    assert err <= tol
    return got


def test_recall_bf16_topk():
    _recall_case(get_config("C2").with_(heads=3), 1e-5)


def test_recall_bf16_mass():
    got = _recall_case(get_config("C2").with_(heads=2), 1e-5, mass_tau=0.6)
    assert got.min() > 0


def test_recall_f32():
    _recall_case(get_config("C1").with_(q_block=64), 1e-5)


def test_recall_g2_inputs_concentrate():
    # 3D-cube token order with smooth Q and K fields: the best 10 % of blocks hold most of the mass
    # (what the recall measures is the selection, here the random-init predictor's)
    _recall_case(get_config("C2").with_(heads=2, generator="g2"), 1e-5)


def test_recall_of_every_block_is_one():
    cfg = get_config("C1").with_(q_block=64)
    inp = make_inputs(cfg, with_grad=False)
    t = {k: to_dev(v) for k, v in inp.items() if k in ("q", "k", "v")}
    b, h = t["q"].shape[:2]
    idx = torch.arange(cfg.nkb, dtype=torch.int32, device="cuda").repeat(b, h, cfg.nqb, 1).contiguous()
    lse = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, q_block=cfg.q_block, kv_block=cfg.kv_block)[1]
    rec = dsv.block_recall(lse, lse, q_block=cfg.q_block)
    assert torch.all(rec == 1.0)
    empty = torch.full_like(lse, -float("inf"))
    assert torch.all(dsv.block_recall(empty, lse, q_block=cfg.q_block) == 0.0)
