"""GPU parity of mass-threshold selection and of attention over ragged block lists.

Selection: the oracle is fed the GPU's own block scores, so the two sides differ only in how the
float32 sums are formed.  Counts must match exactly wherever the oracle's cut is further than
MASS_EPS (relative to the row total) from being decided otherwise -- a bound on the rounding of a
float32 sum of at most 4096 scores (4096 * 2^-24 = 2.4e-4, with slack); nearer the cut the GPU may
take one block more or fewer, but its set must still be the greedy one for its count.
Attention over the ragged lists is held to the same tolerances as top-k lists."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from oracle import dsv_oracle as O
from tests.gpu_helpers import FWD_BF16_MAXABS, FWD_BF16_RELL2, FWD_F32_MAXABS, GRAD_BF16_MAXABS, log, rel_l2, to_dev, to_f64
from workloads import get_config, make_inputs
from workloads.generator import widen

pytestmark = pytest.mark.gpu
MASS_EPS = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsv.load_library()
    yield
    torch.cuda.synchronize()


def _check_selection(idx, cnt, scores, tau, kmax):
    """idx [R, kmax], cnt [R] from the GPU against the oracle on the same float32 scores [R, nkb]."""
    ref_idx, ref_cnt = O.select_mass(scores, tau, kmax)
    margin = O.mass_margin(scores, tau) / np.maximum(scores.sum(-1), 1e-30)
    capped = ref_cnt == kmax
    exact = (margin > MASS_EPS) | capped
    log(f"[parity] mass tau={tau} kmax={kmax}: rows under the exact rule {exact.mean():.3f}, "
        f"counts {ref_cnt.min()}..{ref_cnt.max()}")
    for r in range(scores.shape[0]):
        m = int(cnt[r])
        assert 1 <= m <= kmax
        assert np.all(idx[r, m:] == -1)
        assert np.all(np.diff(idx[r, :m]) > 0)
        if exact[r]:
            assert m == ref_cnt[r] and np.array_equal(idx[r, :m], ref_idx[r, :m]), r
        else:
            assert abs(m - int(ref_cnt[r])) <= 1, r
            assert np.array_equal(idx[r, :m], O.select_topk_row(scores[r], m)), r
    return exact.mean()


@pytest.mark.parametrize("tau,kmax", [(0.9, 128), (0.5, 32), (0.3, 8), (1.0, 128)])
def test_select_mass_matches_the_oracle(tau, kmax):
    cfg = get_config("C2").with_(heads=4)
    inp = make_inputs(cfg, with_grad=False)
    t = {k: to_dev(v) for k, v in inp.items() if k in ("q", "k", "wq", "wk")}
    scores = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], q_block=cfg.q_block, kv_block=cfg.kv_block)
    idx, cnt = dsv.select_mass(scores, tau, kmax, q_block=cfg.q_block, kv_block=cfg.kv_block)
    torch.cuda.synchronize()
    s = to_f64(scores).reshape(-1, cfg.nkb)
    _check_selection(idx.cpu().numpy().reshape(-1, kmax), cnt.cpu().numpy().reshape(-1), s, tau, kmax)


def test_select_mass_on_constructed_rows():
    # rows with exact ties, zeros and one dominant block, at several widths (one wave per row)
    rng = np.random.default_rng(5)
    for nkb in (1, 7, 64, 100, 2048):
        rows = np.abs(rng.integers(0, 4, (12, nkb))).astype(np.float32)
        rows[0] = 0.0
        rows[1, :] = 1.0
        rows[2, nkb // 2] = 1000.0
        scores = torch.from_numpy(rows.reshape(1, 12, 1, nkb)).cuda()
        kmax = max(1, nkb // 2)
        idx, cnt = dsv.select_mass(scores, 0.75, kmax, q_block=64 * nkb, kv_block=64)
        torch.cuda.synchronize()
        _check_selection(idx.cpu().numpy().reshape(-1, kmax), cnt.cpu().numpy().reshape(-1), rows.astype(np.float64),
                         0.75, kmax)


def _ragged_case(cfg, tau, kmax):
    inp = make_inputs(cfg, with_grad=True)
    x = {k: widen(v) for k, v in inp.items()}
    t = {k: to_dev(v) for k, v in inp.items()}
    scores = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], q_block=cfg.q_block, kv_block=cfg.kv_block)
    idx, cnt = dsv.select_mass(scores, tau, kmax, q_block=cfg.q_block, kv_block=cfg.kv_block)
    return x, t, idx, cnt


def _run_attention(cfg, t, idx, cnt):
    res = cfg.dtype == "bf16"
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block, block_counts=cnt)
    out = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, residual=res, **kw)
    grads = dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], out[0], t["do"], out[1], idx, o_lo=out[2] if res else None,
                                **kw)
    torch.cuda.synchronize()
    return out[0], out[1], grads


def _oracle_lists(idx, cnt):
    """The GPU's lists as the oracle reads them: entries past the count become -1 padding."""
    a = idx.cpu().numpy().copy()
    c = np.clip(cnt.cpu().numpy(), 0, a.shape[-1])
    a[np.arange(a.shape[-1]) >= c[..., None]] = -1
    return a


def test_ragged_attention_bf16_matches_the_oracle():
    cfg = get_config("C2").with_(heads=4)
    x, t, idx, cnt = _ragged_case(cfg, 0.5, 96)
    # force a few special rows: an empty list, and counts outside [0, k] (clamped); the row with
    # a count above k gets a full list of k valid blocks, since a count past the selection
    # would point at -1 padding (an out-of-range index, which the kernels clamp)
    cnt[0, 0, 3] = 0
    cnt[0, 1, 5] = -7
    full = np.sort(np.random.default_rng(9).choice(cfg.nkb, 96, replace=False)).astype(np.int32)
    idx[0, 2, 7] = torch.from_numpy(full).to(idx.device)
    cnt[0, 2, 7] = 1000
    lists = _oracle_lists(idx, cnt)
    log(f"[parity] ragged bf16: counts {int(cnt.clamp(0, 96).min())}..{int(cnt.clamp(0, 96).max())}")
    o, lse, grads = _run_attention(cfg, t, idx, cnt)
    sc = 1.0 / np.sqrt(cfg.head_dim)
    o_o, lse_o = O.sparse_attn_fwd(x["q"], x["k"], x["v"], lists, cfg.q_block, cfg.kv_block, sc)
    og = to_f64(o)
    empty = [(0, 0, 3), (0, 1, 5)]
    for h, qb in ((0, 3), (1, 5)):
        rows = slice(qb * cfg.q_block, (qb + 1) * cfg.q_block)
        assert np.all(og[0, h, rows] == 0) and np.all(np.isneginf(to_f64(lse)[0, h, rows]))
        o_o[0, h, rows] = 0.0  # the oracle's softmax over no keys is undefined; the library defines O = 0
        lse_o[0, h, rows] = -np.inf
    err, rl2 = np.abs(og - o_o).max(), rel_l2(og, o_o)
    log(f"[parity] ragged bf16 fwd max-abs {err:.3e} rel-L2 {rl2:.3e} ({len(empty)} empty rows)")
    assert err <= FWD_BF16_MAXABS and rl2 <= FWD_BF16_RELL2
    fin = np.isfinite(lse_o)
    assert np.abs(to_f64(lse)[fin] - lse_o[fin]).max() <= 1e-2
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], lists, cfg.q_block, cfg.kv_block, sc)
    for nm, got, ref in zip(("dq", "dk", "dv"), grads, g_o):
        e = np.abs(to_f64(got) - ref).max()
        log(f"[parity] ragged bf16 {nm} max-abs {e:.3e}")
        assert e <= GRAD_BF16_MAXABS
    for h, qb in ((0, 3), (1, 5)):  # no list, no gradient to its queries
        assert np.all(to_f64(grads[0])[0, h, qb * cfg.q_block:(qb + 1) * cfg.q_block] == 0)


def test_ragged_attention_f32_matches_the_oracle():
    cfg = get_config("C1").with_(q_block=64)
    x, t, idx, cnt = _ragged_case(cfg, 0.6, 8)
    lists = _oracle_lists(idx, cnt)
    o, lse, grads = _run_attention(cfg, t, idx, cnt)
    sc = 1.0 / np.sqrt(cfg.head_dim)
    o_o, lse_o = O.sparse_attn_fwd(x["q"], x["k"], x["v"], lists, cfg.q_block, cfg.kv_block, sc)
    assert np.abs(to_f64(o) - o_o).max() <= FWD_F32_MAXABS
    assert np.abs(to_f64(lse) - lse_o).max() <= FWD_F32_MAXABS
    for got, ref in zip(grads, O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], lists, cfg.q_block, cfg.kv_block, sc)):
        assert np.abs(to_f64(got) - ref).max() <= 1e-4


@pytest.mark.parametrize("dense_above", [0.0, 0.05, 0.3, 0.5, 0.9999])
def test_head_density_matches_the_oracle(dense_above):
    # counts from mass selection on real scores, plus constructed heads: empty, full, out of range
    cfg = get_config("C2").with_(heads=4)
    inp = make_inputs(cfg, with_grad=False)
    t = {k: to_dev(v) for k, v in inp.items() if k in ("q", "k", "wq", "wk")}
    scores = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], q_block=cfg.q_block, kv_block=cfg.kv_block)
    kmax = 96
    _, cnt = dsv.select_mass(scores, 0.5, kmax, q_block=cfg.q_block, kv_block=cfg.kv_block)
    cnt[0, 1] = 0
    cnt[0, 2] = kmax
    cnt[0, 3, ::2] = 1000
    cnt[0, 3, 1::2] = -3
    thr = float(np.float32(dense_above))  # the value the float argument carries
    kw = dict(topk=kmax, seq_len=cfg.seq_len, q_block=cfg.q_block, kv_block=cfg.kv_block, dense_above=thr)
    dens, flag = dsv.head_density(cnt, **kw)
    torch.cuda.synchronize()
    ref_d, ref_f = O.head_density(cnt.cpu().numpy(), kmax, cfg.nqb, cfg.nkb, thr)
    assert np.array_equal(dens.cpu().numpy(), ref_d.astype(np.float32))
    assert np.array_equal(flag.cpu().numpy().astype(bool), ref_f)
    full_d, full_f = dsv.head_density(None, batch=1, heads=4, **kw)
    torch.cuda.synchronize()
    assert np.all(full_d.cpu().numpy() == np.float32(kmax / cfg.nkb))
    log(f"[parity] head density (dense_above={thr}): {dens.cpu().numpy().round(4).tolist()}, flags {flag.cpu().numpy().tolist()}")
