"""Pins of the CPU oracle to facts outside itself (closed forms, library routines,
brute force, finite differences, a hand-worked example, invariants).

Each test is chosen so that a plausible slip in the oracle -- a dropped term, a
wrong sign or index, a transposed operand, a wrong tie rule -- fails it.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import dsv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, k, v, scale, mask=None):
    """torch's scaled_dot_product_attention in float64 on the CPU (a library routine)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale).numpy()


def _random_idx(rng, nqb, nkb, k):
    return np.stack([np.sort(rng.choice(nkb, size=k, replace=False)) for _ in range(nqb)]).astype(np.int32)


def _block_mask(idx, n, bq, bk):
    mask = np.zeros((n, n), dtype=bool)
    for qb, row in enumerate(idx):
        for kb in row:
            mask[qb * bq:(qb + 1) * bq, kb * bk:(kb + 1) * bk] = True
    return mask


# ---------------------------------------------------------------- rounding


def test_round_bf16_matches_torch_on_float32_values():
    rng = _rng(0)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0) ** rng.integers(-30, 30, 20000)
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_hand_cases():
    cases = {
        1.0 + 2.0 ** -8: 1.0,                      # halfway between 1 and 1+2^-7 -> even (1)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,      # halfway between odd and even -> even
        1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7,  # just above halfway -> up
        -(1.0 + 3 * 2.0 ** -8): -(1.0 + 2.0 ** -6),
        2.0 ** -130: 2.0 ** -130,                  # subnormal, representable
        2.0 ** -134: 0.0,                          # half of the smallest subnormal -> even (0)
        3 * 2.0 ** -134: 2.0 ** -132,              # 1.5 quanta -> 2 quanta (even)
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert O.round_bf16(np.array([x]))[0] == want, x
    assert np.isinf(O.round_bf16(np.array([3.4e38]))[0])


def test_project_rounds_to_nearest_bf16_of_exact_product():
    rng = _rng(1)
    x = rng.standard_normal((64, 32))
    w = rng.standard_normal((32, 8))
    exact = x @ w
    got = O.project(x, w, "bf16")
    # every value is a bf16 number, and within half a bf16 ulp of the exact product
    f32 = got.astype(np.float32)
    assert np.all(f32.astype(np.float64) == got)
    assert np.all((f32.view(np.uint32) & 0xFFFF) == 0)
    ulp = np.ldexp(1.0, np.frexp(np.abs(got))[1] - 8)
    assert np.all(np.abs(got - exact) <= 0.5 * ulp + 1e-300)
    np.testing.assert_allclose(O.project(x, w, "f32"), exact, rtol=0, atol=0)


# ---------------------------------------------------------------- forward


def _brute_force_attention(q, k, v, scale):
    n, d = q.shape
    out = []
    for i in range(n):
        logits = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in range(k.shape[0])]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = sum(w)
        out.append([sum(w[j] * v[j][c] for j in range(k.shape[0])) / z for c in range(v.shape[1])])
    return np.array(out)


def test_all_blocks_is_dense_attention_brute_force():
    rng = _rng(2)
    n, d, bq, bk = 128, 8, 32, 32
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    idx = np.tile(np.arange(n // bk, dtype=np.int32), (n // bq, 1))
    o, _ = O.sparse_attn_fwd(q[None, None], k[None, None], v[None, None], idx[None, None], bq, bk, 0.3)
    np.testing.assert_allclose(o[0, 0], _brute_force_attention(q, k, v, 0.3), rtol=0, atol=1e-12)


def test_all_blocks_is_dense_attention_sdpa_c1_shape():
    rng = _rng(3)
    b, h, n, d, bq, bk = 1, 2, 1024, 64, 64, 64
    q, k, v = (rng.standard_normal((b, h, n, d)) for _ in range(3))
    idx = np.tile(np.arange(n // bk, dtype=np.int32), (b, h, n // bq, 1))
    o, _ = O.sparse_attn_fwd(q, k, v, idx, bq, bk, 1 / 8)
    np.testing.assert_allclose(o, _sdpa(q, k, v, 1 / 8), rtol=0, atol=1e-10)


@pytest.mark.parametrize("n,d,bq,bk,k", [(1024, 64, 64, 64, 2), (2048, 64, 128, 64, 13)])
def test_sparse_equals_masked_dense(n, d, bq, bk, k):
    rng = _rng(4 + n)
    q, k_, v = (rng.standard_normal((n, d)) for _ in range(3))
    idx = _random_idx(rng, n // bq, n // bk, k)
    o, _ = O.sparse_attn_fwd(q[None, None], k_[None, None], v[None, None], idx[None, None], bq, bk, 0.125)
    want = _sdpa(q, k_, v, 0.125, _block_mask(idx, n, bq, bk))
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-12)


def test_single_block_constant_keys_is_mean_of_values():
    # k = 1 and all keys of the chosen block equal -> equal logits -> O = mean of that block's V
    rng = _rng(5)
    n, d, bq, bk = 256, 16, 64, 64
    q, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    k[128:192] = k[128]
    idx = np.full((n // bq, 1), 2, dtype=np.int32)
    o, lse = O.sparse_attn_fwd(q[None, None], k[None, None], v[None, None], idx[None, None], bq, bk, 0.7)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[128:192].mean(0), (n, d)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], 0.7 * q @ k[128] + math.log(64), rtol=0, atol=1e-12)


def test_lse_matches_scipy_logsumexp():
    rng = _rng(6)
    n, d, bq, bk, kk = 512, 32, 64, 64, 3
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    idx = _random_idx(rng, n // bq, n // bk, kk)
    _, lse = O.sparse_attn_fwd(q[None, None], k[None, None], v[None, None], idx[None, None], bq, bk, 0.2)
    for qb in range(n // bq):
        keys = np.concatenate([np.arange(j * bk, (j + 1) * bk) for j in idx[qb]])
        want = scipy.special.logsumexp(0.2 * q[qb * bq:(qb + 1) * bq] @ k[keys].T, axis=1)
        np.testing.assert_allclose(lse[0, 0, qb * bq:(qb + 1) * bq], want, rtol=0, atol=1e-12)


def test_sparse_weights_rows_sum_to_one_and_order_of_list_is_irrelevant():
    rng = _rng(7)
    n, d, bq, bk, kk = 256, 16, 64, 32, 3
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    idx = _random_idx(rng, n // bq, n // bk, kk)
    o1, l1 = O.sparse_attn_fwd(q[None, None], k[None, None], v[None, None], idx[None, None], bq, bk, 0.3)
    o2, l2 = O.sparse_attn_fwd(q[None, None], k[None, None], v[None, None], idx[None, None, :, ::-1], bq, bk, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    # V = all-ones -> O = all-ones iff the sparse weights of every row sum to 1
    ones = np.ones_like(v)
    o3, _ = O.sparse_attn_fwd(q[None, None], k[None, None], ones[None, None], idx[None, None], bq, bk, 0.3)
    np.testing.assert_allclose(o3, 1.0, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- backward


def test_backward_matches_central_finite_differences():
    rng = _rng(8)
    n, d, bq, bk, kk, sc = 128, 16, 32, 32, 2, 0.25
    q, k, v, do = (rng.standard_normal((1, 1, n, d)) for _ in range(4))
    idx = _random_idx(rng, n // bq, n // bk, kk)[None, None]

    def loss(q_, k_, v_):
        o, _ = O.sparse_attn_fwd(q_, k_, v_, idx, bq, bk, sc)
        return float((o * do).sum())

    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, bq, bk, sc)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        flat, nflat = x.reshape(-1), num.reshape(-1)
        for t in range(flat.size):
            old = flat[t]
            flat[t] = old + h
            lp = loss(q, k, v)
            flat[t] = old - h
            lm = loss(q, k, v)
            flat[t] = old
            nflat[t] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-6, (name, err)


def test_backward_matches_torch_autograd_masked_dense():
    rng = _rng(9)
    b, h, n, d, bq, bk, kk, sc = 1, 2, 512, 32, 64, 32, 4, 0.17
    q, k, v, do = (rng.standard_normal((b, h, n, d)) for _ in range(4))
    idx = np.stack([_random_idx(rng, n // bq, n // bk, kk) for _ in range(h)])[None]
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, bq, bk, sc)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    mask = torch.from_numpy(np.stack([_block_mask(idx[0, hh], n, bq, bk) for hh in range(h)])[None])
    s = sc * tq @ tk.transpose(-1, -2)
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    (o * torch.from_numpy(do)).sum().backward()
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-10)


def test_kv_block_gradient_equals_full_backward_slice():
    rng = _rng(10)
    n, d, bq, bk, kk, sc = 512, 16, 64, 32, 5, 0.3
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    idx = _random_idx(rng, n // bq, n // bk, kk)
    _, dk, dv = O.sparse_attn_bwd(q[None, None], k[None, None], v[None, None], do[None, None],
                                  idx[None, None], bq, bk, sc)
    for kb in (0, 3, 7, 15):
        gk, gv = O.attn_bwd_kvblock(q, k, v, do, idx, kb, bq, bk, sc)
        np.testing.assert_allclose(gk, dk[0, 0, kb * bk:(kb + 1) * bk], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gv, dv[0, 0, kb * bk:(kb + 1) * bk], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- predictor


def test_identity_predictor_gives_true_block_mass():
    # r = d, W = I, pred_scale = sm_scale, no rounding: the score is the block sum of the
    # exact dense attention matrix (torch softmax in float64), and the selection is its top-k.
    rng = _rng(11)
    b, h, n, d, bq, bk, kk, sc = 1, 2, 1024, 16, 64, 64, 3, 0.25
    q, k = rng.standard_normal((b, h, n, d)), rng.standard_normal((b, h, n, d))
    eye = np.tile(np.eye(d), (h, 1, 1))
    scores, _, _ = O.predict(q, k, eye, eye, bq, bk, sc, "f32")
    p = torch.softmax(sc * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2), dim=-1)
    mass = p.reshape(b, h, n // bq, bq, n // bk, bk).sum(dim=(3, 5)).numpy()
    np.testing.assert_allclose(scores, mass, rtol=0, atol=1e-12)
    idx = O.select_topk(scores, kk)
    for hh in range(h):
        for qb in range(n // bq):
            top = sorted(range(n // bk), key=lambda j: (-mass[0, hh, qb, j], j))[:kk]
            assert list(idx[0, hh, qb]) == sorted(top)


def test_predictor_projections_are_applied_to_the_right_operands():
    # scores(q, k, A, B) == scores(q @ A, k @ B, I, I): catches a swap of Wq and Wk or of q and k
    rng = _rng(12)
    n, d, r, bq, bk = 512, 16, 8, 64, 64
    q, k = rng.standard_normal((1, 1, n, d)), rng.standard_normal((1, 1, n, d))
    a, bm = rng.standard_normal((1, d, r)), rng.standard_normal((1, d, r))
    s1, ql, kl = O.predict(q, k, a, bm, bq, bk, 0.3, "f32")
    eye = np.eye(r)[None]
    s2, _, _ = O.predict(q @ a[0], k @ bm[0], eye, eye, bq, bk, 0.3, "f32")
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-12)
    s3, _, _ = O.predict(q @ bm[0], k @ a[0], eye, eye, bq, bk, 0.3, "f32")
    assert np.abs(s1 - s3).max() > 1e-3
    # the score is not symmetric in (q, k): swapping the roles changes it
    s4, _, _ = O.predict(k, q, a, bm, bq, bk, 0.3, "f32")
    assert np.abs(s1 - s4).max() > 1e-3


def test_score_rows_sum_to_block_size_and_are_nonnegative():
    rng = _rng(13)
    n, d, r, bq, bk = 1024, 32, 16, 128, 64
    q, k = rng.standard_normal((1, 2, n, d)) * 3, rng.standard_normal((1, 2, n, d)) * 3
    w1, w2 = rng.standard_normal((2, d, r)), rng.standard_normal((2, d, r))
    s, _, _ = O.predict(q, k, w1, w2, bq, bk, 0.5, "bf16")
    assert np.all(s >= 0)
    np.testing.assert_allclose(s.sum(-1), bq, rtol=0, atol=1e-10)


def test_bf16_query_operand_carries_the_scale_before_its_rounding():
    # R3: the query operand is bf16(pred_scale * log2(e) * Q Wq).  With pred_scale * log2(e) a
    # power of two the scaling commutes with the rounding, so the bf16 predictor must equal the
    # textbook predicted mass of pred_scale * <bf16(Q Wq), bf16(K Wk)> (float64 torch softmax over
    # every key, then block sums; bf16 rounding by torch's own cast).  This catches a scale applied
    # twice or not at all, logits left in base-2 units, and a rounding in the wrong place.
    rng = _rng(16)
    n, d, r, bq, bk = 512, 32, 8, 64, 64
    q, k = rng.standard_normal((1, 2, n, d)) * 2, rng.standard_normal((1, 2, n, d)) * 2
    wq, wk = rng.standard_normal((2, d, r)), rng.standard_normal((2, d, r))
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).double()
    ps = 0.125 * math.log(2.0)  # pred_scale * log2(e) = 2^-3
    s, qt, kl = O.predict(q, k, wq, wk, bq, bk, ps, "bf16")
    for h in range(2):
        ql, kk = bf(q[0, h] @ wq[h]), bf(k[0, h] @ wk[h])
        p = torch.softmax(ps * ql @ kk.T, dim=-1)
        mass = p.reshape(n // bq, bq, n // bk, bk).sum(dim=(1, 3)).numpy()
        np.testing.assert_allclose(s[0, h], mass, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(qt[0, h], (0.125 * ql).numpy())
    # any other scale: the operand is the rounding of the scaled product (not the scaled rounding)
    ps = 0.3
    _, qt, _ = O.predict(q, k, wq, wk, bq, bk, ps, "bf16")
    y = ps / math.log(2.0) * (q[0, 0] @ wq[0])
    np.testing.assert_array_equal(qt[0, 0], bf(y).numpy())
    assert np.any(qt[0, 0] != ps / math.log(2.0) * bf(q[0, 0] @ wq[0]).numpy())


@pytest.mark.parametrize("generator", ["g1", "g2"])
def test_bf16_scores_lie_within_two_operand_roundings_of_the_exact_mass(generator):
    # R3 at the default, non-power-of-two scale, pinned to the unrounded predictor rather than to
    # the oracle's own formula.  Exact fp64 logits: l*_ij = pred_scale <a_i, b_j>, a = Q Wq,
    # b = K Wk.  Rounding each operand once to bf16 (8 significant bits: relative error at most
    # u = 2^-8 for these normal-range values) moves a logit by D_ij with
    #   |D_ij| <= E_ij = pred_scale sum_c |a_ic b_jc| (2u + u^2).
    # With P* the exact softmax, P_ij = P*_ij exp(D_ij) / Z_i and Z_i = sum_j P*_ij exp(D_ij) lies in
    # [sum_j P*_ij exp(-E_ij), sum_j P*_ij exp(E_ij)], so a block score sum_{i in qb, j in kb} P_ij
    # lies between sum P*_ij exp(-E_ij) / Zhi_i and sum P*_ij exp(E_ij) / Zlo_i.
    from workloads import get_config, make_inputs
    from workloads.generator import widen

    cfg = get_config("C2").with_(heads=2, latent=(4, 16, 16), generator=generator)  # N = 1024, d = 64, r = 16
    x = {nm: widen(a) for nm, a in make_inputs(cfg, with_grad=False).items()}
    ps = 1.0 / math.sqrt(cfg.head_dim)
    bq, bk = cfg.q_block, cfg.kv_block
    s, qt, kl = O.predict(x["q"], x["k"], x["wq"], x["wk"], bq, bk, ps, "bf16")
    u = 2.0 ** -8
    n = cfg.seq_len
    blocks = lambda m: m.reshape(n // bq, bq, n // bk, bk).sum(axis=(1, 3))
    for h in range(cfg.heads):
        a, b = x["q"][0, h] @ x["wq"][h], x["k"][0, h] @ x["wk"][h]
        exact = torch.softmax(torch.from_numpy(ps * a @ b.T), dim=-1).numpy()     # P*, float64
        e = ps * (np.abs(a) @ np.abs(b).T) * (2 * u + u * u) * (1 + 1e-12)     # E_ij (+ fp64 slack)
        zlo = (exact * np.exp(-e)).sum(axis=1, keepdims=True)
        zhi = (exact * np.exp(e)).sum(axis=1, keepdims=True)
        lo, hi = blocks(exact * np.exp(-e) / zhi), blocks(exact * np.exp(e) / zlo)
        within = lambda sc: bool(np.all((sc >= lo - 1e-12) & (sc <= hi + 1e-12)))
        assert within(s[0, h]), (s[0, h] - hi).max()
        err, slack = np.abs(s[0, h] - blocks(exact)), np.maximum(hi - blocks(exact), blocks(exact) - lo)
        print(f"{generator} h={h}: max |score - exact| {err.max():.3e}, max half-width {slack.max():.3e}")
        assert err.max() > 0  # the operands are rounded: the scores move
        # the operands are bf16 values within u of the exact scaled projections
        y = ps / math.log(2.0) * a
        np.testing.assert_array_equal(qt[0, h], O.round_bf16(qt[0, h]))
        np.testing.assert_array_equal(kl[0, h], O.round_bf16(kl[0, h]))
        assert np.all(np.abs(qt[0, h] - y) <= u * np.abs(y)) and np.all(np.abs(kl[0, h] - b) <= u * np.abs(b))
        # planted slips (in the oracle's score step, on the CPU) fall outside the bound: logits left
        # in base-2 units, the log scale applied twice, the key operand never projected by Wk's scale
        # (a factor 2 on K_lr)
        ql, kk = qt[0, h], kl[0, h]
        assert not within(O.block_scores_head(ql, kk, bq, bk, 1.0))
        assert not within(O.block_scores_head(ql, kk, bq, bk, O.LN2 * O.LN2))
        assert not within(O.block_scores_head(ql, 2 * kk, bq, bk, O.LN2))


def test_representative_scores_are_the_one_row_softmax():
    rng = _rng(14)
    n, r, bq, bk = 256, 8, 64, 32
    ql, kl = rng.standard_normal((n, r)), rng.standard_normal((n, r))
    s = O.representative_scores_head(ql, kl, bq, bk, 0.4, rep=0)
    for qb in range(n // bq):
        row = scipy.special.softmax(0.4 * kl @ ql[qb * bq])
        np.testing.assert_allclose(s[qb], row.reshape(-1, bk).sum(1), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- selection


def test_selection_against_python_sort_with_ties():
    rng = _rng(15)
    for trial in range(200):
        nkb = int(rng.integers(1, 300))
        k = int(rng.integers(1, nkb + 1))
        s = rng.integers(0, 6, nkb).astype(np.float64) * 0.25  # many exact ties
        if trial % 3 == 0:
            s = rng.random(nkb)
        got = O.select_topk_row(s, k)
        want = sorted(sorted(range(nkb), key=lambda j: (-s[j], j))[:k])
        assert list(got) == want
        # invariants: ascending, distinct, every kept score >= every dropped score,
        # and among equal scores at the boundary the kept indices are the smaller ones
        assert np.all(np.diff(got) > 0)
        kept = np.zeros(nkb, bool)
        kept[got] = True
        if k < nkb:
            assert s[kept].min() >= s[~kept].max()
            t = s[kept].min()
            tied_kept = np.nonzero(kept & (s == t))[0]
            tied_drop = np.nonzero(~kept & (s == t))[0]
            if tied_drop.size:
                assert tied_kept.max() < tied_drop.min()


def test_topk_gap():
    s = np.array([[0.1, 0.5, 0.3, 0.3, 0.05]])
    # sorted descending: 0.5, 0.3, 0.3, 0.1, 0.05
    np.testing.assert_allclose(O.topk_gap(s, 1), [0.2])
    np.testing.assert_allclose(O.topk_gap(s, 2), [0.0])
    np.testing.assert_allclose(O.topk_gap(s, 3), [0.2])
    assert np.isinf(O.topk_gap(s, 5)[0])


# ---------------------------------------------------------------- whole step


def test_hand_worked_golden_example():
    g = json.load(open(os.path.join(GOLDEN, "uniform_logits_n8.json")))
    arr = lambda key: np.array(g[key], dtype=np.float64)[None, None]
    res = O.dsv_step(arr("q"), arr("k"), arr("v"), arr("do"), np.array(g["wq"], float)[None],
                     np.array(g["wk"], float)[None], g["q_block"], g["kv_block"], g["topk"], "f32",
                     sm_scale=g["sm_scale"], pred_scale=g["pred_scale"])
    e = g["expected"]
    np.testing.assert_allclose(res["scores"][0, 0], e["scores"], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(res["idx"][0, 0], e["idx"])
    np.testing.assert_allclose(res["o"][0, 0], e["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(res["lse"][0, 0], e["lse"], rtol=0, atol=1e-15)
    dq, dk, dv = res["grads"]
    np.testing.assert_allclose(dq[0, 0], e["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], e["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], e["dv"], rtol=0, atol=1e-14)


def test_heads_are_independent_and_permutation_equivariant():
    rng = _rng(16)
    b, h, n, d, r, bq, bk, kk = 1, 3, 256, 16, 8, 64, 32, 3
    q, k, v, do = (rng.standard_normal((b, h, n, d)) for _ in range(4))
    wq, wk = rng.standard_normal((h, d, r)), rng.standard_normal((h, d, r))
    res = O.dsv_step(q, k, v, do, wq, wk, bq, bk, kk, "bf16")
    perm = [2, 0, 1]
    res_p = O.dsv_step(q[:, perm], k[:, perm], v[:, perm], do[:, perm], wq[perm], wk[perm], bq, bk, kk, "bf16")
    for key in ("scores", "idx", "o", "lse"):
        np.testing.assert_array_equal(res_p[key], res[key][:, perm])
    for g1, g2 in zip(res_p["grads"], res["grads"]):
        np.testing.assert_array_equal(g1, g2[:, perm])
    # one head alone gives the same result as inside the batch
    one = O.dsv_step(q[:, 1:2], k[:, 1:2], v[:, 1:2], do[:, 1:2], wq[1:2], wk[1:2], bq, bk, kk, "bf16")
    np.testing.assert_array_equal(one["idx"], res["idx"][:, 1:2])
    np.testing.assert_array_equal(one["o"], res["o"][:, 1:2])


def test_rejects_bad_block_sizes():
    z = np.zeros((1, 1, 100, 4))
    with pytest.raises(ValueError):
        O.sparse_attn_fwd(z, z, z, np.zeros((1, 1, 1, 1), np.int32), 64, 64, 1.0)


# ------------------------------------------------------------------ mass-threshold selection (R13)


def _greedy_mass_python(scores, tau, kmax):
    """Independent statement of R13 with Python's sort and a running sum."""
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
    target, acc, chosen = tau * sum(scores), 0.0, []
    for i in order:
        if len(chosen) == kmax or (chosen and acc >= target):
            break
        chosen.append(i)
        acc += scores[i]
    return sorted(chosen)


def test_mass_selection_is_the_smallest_set_reaching_the_target():
    import itertools
    rng = np.random.default_rng(7)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        s = rng.integers(0, 6, n).astype(np.float64)  # small integers: exact sums, many ties
        if s.sum() == 0:
            s[0] = 1.0
        tau = float(rng.choice([0.01, 0.3, 0.5, 0.75, 0.9, 1.0]))
        sel = O.select_mass_row(s, tau, n)
        target = tau * s.sum()
        assert s[sel].sum() >= target
        best = min(m for m in range(1, n + 1)
                   if any(s[list(c)].sum() >= target for c in itertools.combinations(range(n), m)))
        assert sel.size == best, (s, tau, sel)
        assert list(sel) == _greedy_mass_python(list(s), tau, n)
        kmax = int(rng.integers(1, n + 1))
        assert list(O.select_mass_row(s, tau, kmax)) == _greedy_mass_python(list(s), tau, kmax)


def test_mass_selection_special_cases():
    s = np.array([2.0, 7.0, 7.0, 0.0, 1.0, 3.0])
    assert list(O.select_mass_row(s, 1e-6, 6)) == [1]              # one block: the top, ties to smaller index
    assert list(O.select_mass_row(s, 1.0, 6)) == [0, 1, 2, 4, 5]   # every nonzero block, the empty one left out
    for k in range(1, 6):                                         # capped below the 5 needed: the top-k rule
        assert np.array_equal(O.select_mass_row(s, 1.0, k), O.select_topk_row(s, k))
    idx, cnt = O.select_mass(np.stack([s, s[::-1]])[None], 0.5, 4)
    assert idx.shape == (1, 2, 4) and list(cnt[0]) == [2, 2]
    assert list(idx[0, 0]) == [1, 2, -1, -1] and list(idx[0, 1]) == [3, 4, -1, -1]
    # the cut at 0.5 * 20 = 10: c_1 = 7 < 10 <= c_2 = 14 -> margin min(14 - 10, 10 - 7) = 3
    assert O.mass_margin(s[None], 0.5)[0] == 3.0


def test_padded_block_lists_select_nothing_extra():
    rng = np.random.default_rng(3)
    n, d, bq, bk = 256, 16, 64, 64
    q, k, v, do = (rng.standard_normal((1, 1, n, d)) for _ in range(4))
    full = np.array([[[[2, 0], [1, 3], [3, 2], [0, 1]]]], np.int32)
    padded = np.concatenate([full, np.full((1, 1, 4, 2), -1, np.int32)], axis=-1)
    o1, l1 = O.sparse_attn_fwd(q, k, v, full, bq, bk, 0.25)
    o2, l2 = O.sparse_attn_fwd(q, k, v, padded, bq, bk, 0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for a, b in zip(O.sparse_attn_bwd(q, k, v, do, full, bq, bk, 0.25), O.sparse_attn_bwd(q, k, v, do, padded, bq, bk, 0.25)):
        assert np.array_equal(a, b)


def test_attention_is_defined_only_for_distinct_in_range_lists():
    # R7 and the block-list contract: a list names each selected block once, within [0, N/Bk);
    # negative entries are padding (R13).  A repeated or out-of-range entry is refused by the
    # forward and the backward alike (the GPU leaves such lists unspecified and can check them).
    rng = _rng(31)
    n, d, bq, bk = 256, 8, 64, 64
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    good = np.array([0, 3, -1], np.int32)
    O.attn_fwd_qblock(q[:bq], k, v, good, bk, 0.5)
    O.attn_bwd_qblock(q[:bq], k, v, do[:bq], good, bk, 0.5)
    for bad in (np.array([1, 1], np.int32), np.array([0, 4], np.int32), np.array([2, -1, 2], np.int32)):
        with pytest.raises(ValueError):
            O.attn_fwd_qblock(q[:bq], k, v, bad, bk, 0.5)
        with pytest.raises(ValueError):
            O.attn_bwd_qblock(q[:bq], k, v, do[:bq], bad, bk, 0.5)
        with pytest.raises(ValueError):
            O.sparse_attn_fwd(q[None, None], k[None, None], v[None, None], np.tile(bad, (1, 1, n // bq, 1)), bq, bk, 0.5)


def test_empty_block_list_defines_zero_output_and_gradient():
    rng = np.random.default_rng(4)
    n, d, bq, bk = 128, 8, 64, 64
    q, k, v, do = (rng.standard_normal((1, 1, n, d)) for _ in range(4))
    idx = np.array([[[[1, -1], [-1, -1]]]], np.int32)  # query block 1 selects nothing
    o, lse = O.sparse_attn_fwd(q, k, v, idx, bq, bk, 0.3)
    assert np.all(o[0, 0, 64:] == 0) and np.all(np.isneginf(lse[0, 0, 64:]))
    o1, _ = O.attn_fwd_qblock(q[0, 0, :64], k[0, 0], v[0, 0], np.array([1]), bk, 0.3)
    assert np.array_equal(o[0, 0, :64], o1)
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, bq, bk, 0.3)
    assert np.all(dq[0, 0, 64:] == 0) and np.all(dk[0, 0, :64] == 0) and np.all(dv[0, 0, :64] == 0)
    gk, gv = O.attn_bwd_kvblock(q[0, 0], k[0, 0], v[0, 0], do[0, 0], idx[0, 0], 1, bq, bk, 0.3)
    assert np.allclose(gk, dk[0, 0, 64:]) and np.allclose(gv, dv[0, 0, 64:])


# ------------------------------------------------------------------ packing for sequence sharding


def test_packing_moves_exactly_the_union_and_attention_is_unchanged():
    rng = np.random.default_rng(11)
    n, d, bq, bk, k = 512, 8, 64, 32, 4
    nqb, nkb = n // bq, n // bk
    q, kk, v = (rng.standard_normal((1, 2, n, d)) for _ in range(3))
    idx = np.stack([np.stack([np.sort(rng.choice(nkb, k, replace=False)) for _ in range(nqb)]) for _ in range(2)])[None]
    counts = rng.integers(0, k + 1, (1, 2, nqb)).astype(np.int32)
    qb0, qb1 = 2, 6
    blocks, count, remapped = O.pack_selected(idx, counts, qb0, qb1, nkb)
    for h in range(2):
        want = set()
        for qb in range(qb0, qb1):
            want |= set(int(x) for x in idx[0, h, qb, :counts[0, h, qb]])
        assert list(blocks[0, h, :count[0, h]]) == sorted(want) and np.all(blocks[0, h, count[0, h]:] == -1)
        for qb in range(qb0, qb1):
            c = counts[0, h, qb]
            assert np.array_equal(blocks[0, h][remapped[0, h, qb - qb0, :c]], idx[0, h, qb, :c])
            assert np.all(remapped[0, h, qb - qb0, c:] == -1)
    kp, vp = O.pack_rows(kk, blocks, count, bk), O.pack_rows(v, blocks, count, bk)
    # attention of the shard's query blocks over the packed buffer equals the original
    rows = slice(qb0 * bq, qb1 * bq)
    shard_idx = np.where(np.arange(k)[None, None, None, :] < counts[:, :, qb0:qb1, None], idx[:, :, qb0:qb1], -1)
    o_ref, l_ref = O.sparse_attn_fwd(q[:, :, rows], kk, v, shard_idx, bq, bk, 0.3)
    o_p, l_p = O.sparse_attn_fwd(q[:, :, rows], kp, vp, remapped, bq, bk, 0.3)
    assert np.array_equal(o_ref, o_p) and np.array_equal(l_ref, l_p)


# ------------------------------------------------------------------ recall of a selection


def test_block_recall_special_cases_and_identity_predictor():
    rng = np.random.default_rng(21)
    n, d, bq, bk = 256, 8, 64, 32
    q, k = (rng.standard_normal((1, 1, n, d)) for _ in range(2))
    nqb, nkb = n // bq, n // bk
    everything = np.tile(np.arange(nkb, dtype=np.int32), (1, 1, nqb, 1))
    np.testing.assert_allclose(O.block_recall(q, k, everything, bq, bk, 0.4), 1.0, rtol=1e-14)
    # one block: the true block mass from the identity predictor (r = d, W = I), per row
    true_mass = O.block_scores_head(q[0, 0], k[0, 0], bq, bk, 0.4)  # sums over the Bq rows
    for kb in (0, 5):
        one = np.full((1, 1, nqb, 1), kb, np.int32)
        np.testing.assert_allclose(O.block_recall(q, k, one, bq, bk, 0.4)[0, 0], true_mass[:, kb] / bq, rtol=1e-12)
    # additivity over disjoint lists, and nothing selected gives 0
    a = np.tile(np.array([1, 6], np.int32), (1, 1, nqb, 1))
    b = np.tile(np.array([0, 3], np.int32), (1, 1, nqb, 1))
    both = np.concatenate([a, b], axis=-1)
    np.testing.assert_allclose(O.block_recall(q, k, both, bq, bk, 0.4),
                               O.block_recall(q, k, a, bq, bk, 0.4) + O.block_recall(q, k, b, bq, bk, 0.4), rtol=1e-12)
    assert np.all(O.block_recall(q, k, np.full((1, 1, nqb, 1), -1, np.int32), bq, bk, 0.4) == 0)


def test_head_density_worked_example():
    # R14 by hand: lists of lengths 1, 2, 3, 4 (clamped to k = 3) over 4 query blocks x 8 KV blocks
    counts = np.array([[[1, 2, 3, 4], [-5, 0, 0, 3]]])
    dens, dense = O.head_density(counts, 3, 4, 8, 0.28)
    assert dens[0, 0] == 9 / 32 and dens[0, 1] == 3 / 32
    assert bool(dense[0, 0]) and not bool(dense[0, 1])          # 9 > floor(8.96) = 8;  3 <= 8
    _, dense = O.head_density(counts, 3, 4, 8, 0.3)
    assert not bool(dense[0, 0])                                # 9 > floor(9.6) = 9 is false
    # full lists: density k / nkb; never dense above 1, always dense below k / nkb
    full = np.full((2, 3, 16), 5)
    dens, dense = O.head_density(full, 5, 16, 40, 1.0)
    assert np.all(dens == 5 / 40) and not dense.any()
    assert O.head_density(full, 5, 16, 40, 0.1)[1].all()
