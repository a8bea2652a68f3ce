"""Power-of-two scaling through the fp16 products of the attention kernels.

The training forward's P V and the dQ kernel's S and dQ products run on fp16 copies of V, K and Q
scaled per head by 2^s (s from the head's largest magnitude), and on dS scaled per row by 2^r;
every scale is a power of two and is undone exactly.  Attention is homogeneous in V and in dO and
unchanged under Q -> 2^a Q, K -> 2^-a K, so scaling inputs by powers of two must scale the outputs
bit for bit -- a wrong shift, a dropped unscale or a scale applied twice breaks the equality.
One more case runs a non-default softmax scale against the oracle."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from oracle import dsv_oracle as O
from tests.gpu_helpers import FWD_BF16_MAXABS, GRAD_BF16_MAXABS, log, to_dev, to_f64
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


def _lists(cfg, seed=3):
    """Random valid block lists (ascending, distinct), [1, H, nqb, k]."""
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(cfg.nkb, cfg.topk, replace=False)) for _ in range(cfg.heads * cfg.nqb)])
    return idx.reshape(1, cfg.heads, cfg.nqb, cfg.topk).astype(np.int32)


def _run(cfg, q, k, v, do, idx, sm_scale=None):
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block, sm_scale=sm_scale)
    o, lse, o_lo = dsv.sparse_attn_fwd(q, k, v, idx, residual=True, **kw)
    dq, dk, dv = dsv.sparse_attn_bwd(q, k, v, o, do, lse, idx, o_lo=o_lo, **kw)
    torch.cuda.synchronize()
    return dict(o=o, o_lo=o_lo, lse=lse, dq=dq, dk=dk, dv=dv)


@pytest.fixture(scope="module")
def case():
    cfg = get_config("C2").with_(heads=2)
    inp = make_inputs(cfg, with_grad=True)
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "do")}
    idx = to_dev(_lists(cfg))
    return cfg, inp, t, idx, _run(cfg, t["q"], t["k"], t["v"], t["do"], idx)


def _same(got, want, name):
    assert torch.equal(got, want), f"{name}: max |diff| {(got.float() - want.float()).abs().max().item():.3e}"


def test_v_scaled_by_2_pow_30(case):
    cfg, _, t, idx, base = case
    s = 2.0 ** 30
    r = _run(cfg, t["q"], t["k"], t["v"] * s, t["do"], idx)
    log("[parity] V * 2^30: outputs scale exactly")
    _same(r["lse"], base["lse"], "lse")
    for n in ("o", "o_lo", "dq", "dk"):
        _same(r[n], base[n] * s, n)
    _same(r["dv"], base["dv"], "dv")


def test_tiny_output_gradient(case):
    cfg, _, t, idx, base = case
    s = 2.0 ** -60  # training gradients are small: dS must not underflow the fp16 product
    r = _run(cfg, t["q"], t["k"], t["v"], t["do"] * s, idx)
    log("[parity] dO * 2^-60: gradients scale exactly")
    for n in ("o", "o_lo", "lse"):
        _same(r[n], base[n], n)
    for n in ("dq", "dk", "dv"):
        _same(r[n], base[n] * s, n)


def test_q_up_k_down(case):
    cfg, _, t, idx, base = case
    a = 2.0 ** 20
    r = _run(cfg, t["q"] * a, t["k"] / a, t["v"], t["do"], idx)
    log("[parity] Q * 2^20, K * 2^-20: logits unchanged, dQ / 2^20, dK * 2^20")
    for n in ("o", "o_lo", "lse", "dv"):
        _same(r[n], base[n], n)
    _same(r["dq"], base["dq"] / a, "dq")
    _same(r["dk"], base["dk"] * a, "dk")


def test_non_default_softmax_scale_matches_the_oracle(case):
    cfg, inp, t, idx, _ = case
    sc = 0.05
    r = _run(cfg, t["q"], t["k"], t["v"], t["do"], idx, sm_scale=sc)
    x = {n: widen(inp[n]) for n in ("q", "k", "v", "do")}
    lists = idx.cpu().numpy()
    o_o, lse_o = O.sparse_attn_fwd(x["q"], x["k"], x["v"], lists, cfg.q_block, cfg.kv_block, sc)
    assert np.abs(to_f64(r["o"]) - o_o).max() <= FWD_BF16_MAXABS
    assert np.abs(to_f64(r["lse"]) - lse_o).max() <= 1e-2
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], lists, cfg.q_block, cfg.kv_block, sc)
    for n, ref in zip(("dq", "dk", "dv"), g_o):
        e = np.abs(to_f64(r[n]) - ref).max()
        log(f"[parity] sm_scale={sc} {n} max-abs {e:.3e}")
        assert e <= GRAD_BF16_MAXABS
