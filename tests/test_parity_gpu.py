"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs.  Criteria: block indices bit-exact wherever the oracle's top-k gap
exceeds 1e-3 (near-ties must be valid choices); with the oracle's indices fed in,
forward max-abs <= 1e-5 (fp32) or <= 2e-2 with relative L2 <= 5e-3 (bf16);
bf16 gradients max-abs <= 3e-2."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from oracle import dsv_oracle as O
from tests.gpu_helpers import (FWD_BF16_MAXABS, bf16_ulp, FWD_BF16_RELL2, FWD_F32_MAXABS, GRAD_BF16_MAXABS, check_indices, log,
                               rel_l2, seeded_idx, to_dev, to_f64)
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


def _scale(d):
    return 1.0 / np.sqrt(d)


def _run_gpu_path(cfg, inp, idx_fed=None, residual=True):
    """predict -> select (GPU); forward/backward with `idx_fed` (or the GPU's own selection).

    bf16 runs hand the forward's O residual to the backward unless residual=False."""
    t = {k: to_dev(v) for k, v in inp.items()}
    scores, qlr, klr = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], q_block=cfg.q_block, kv_block=cfg.kv_block,
                                   return_projections=True)
    idx = dsv.select_topk(scores, cfg.topk, q_block=cfg.q_block, kv_block=cfg.kv_block)
    use = idx if idx_fed is None else to_dev(idx_fed)
    res = residual and cfg.dtype == "bf16"
    out = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], use, q_block=cfg.q_block, kv_block=cfg.kv_block, residual=res)
    o, lse = out[0], out[1]
    o_lo = out[2] if res else None
    grads = None
    if "do" in t:
        grads = dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, use, q_block=cfg.q_block,
                                    kv_block=cfg.kv_block, o_lo=o_lo)
    torch.cuda.synchronize()
    return dict(t=t, scores=scores, qlr=qlr, klr=klr, idx=idx, o=o, lse=lse, o_lo=o_lo, grads=grads)


# ------------------------------------------------------------------ C1: tiny fp32, full path


def test_c1_fp32_full_path():
    cfg = get_config("C1")
    log(f"[parity] C1 fp32 N={cfg.seq_len} H={cfg.heads}")
    inp = make_inputs(cfg, with_grad=True)
    x = {k: widen(v) for k, v in inp.items()}
    sc = _scale(cfg.head_dim)
    scores_o, qlr_o, klr_o = O.predict(x["q"], x["k"], x["wq"], x["wk"], cfg.q_block, cfg.kv_block, sc, "f32")
    idx_o = O.select_topk(scores_o, cfg.topk)
    o_o, lse_o = O.sparse_attn_fwd(x["q"], x["k"], x["v"], idx_o, cfg.q_block, cfg.kv_block, sc)
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], idx_o, cfg.q_block, cfg.kv_block, sc)
    r = _run_gpu_path(cfg, inp, idx_fed=idx_o)
    np.testing.assert_allclose(to_f64(r["qlr"]), qlr_o, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(to_f64(r["scores"]), scores_o, rtol=1e-4, atol=1e-5)
    cov = check_indices(r["idx"].cpu().numpy(), scores_o, cfg.topk)
    log(f"[parity] C1 index coverage {cov:.3f}")
    assert np.abs(to_f64(r["o"]) - o_o).max() <= FWD_F32_MAXABS
    assert np.abs(to_f64(r["lse"]) - lse_o).max() <= FWD_F32_MAXABS
    for got, ref in zip(r["grads"], g_o):
        assert np.abs(to_f64(got) - ref).max() <= 1e-4


# ------------------------------------------------------------------ selection alone, bit-exact


@pytest.mark.parametrize("b,h,nqb,nkb,k", [(1, 2, 16, 16, 2), (1, 3, 128, 128, 13), (2, 2, 64, 1024, 103),
                                           (1, 2, 64, 2048, 205), (1, 1, 8, 4096, 4096), (1, 1, 4, 100, 1),
                                           (1, 1, 4, 100, 100), (1, 1, 4, 100, 37)])
def test_select_matches_oracle_bit_exactly(b, h, nqb, nkb, k):
    log(f"[parity] select nkb={nkb} k={k}")
    rng = np.random.default_rng(nkb + k)
    s = rng.random((b, h, nqb, nkb)).astype(np.float32)
    s[..., ::7] = np.float32(0.5)  # many exact ties
    s[0, 0, 0] = 0.0               # an all-zero row
    idx = dsv.select_topk(to_dev(s), k, q_block=nkb * 64 // nqb, kv_block=64)
    want = O.select_topk(s.astype(np.float64), k)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)


# ------------------------------------------------------------------ bf16 configs, full oracle on sampled heads


def _bf16_config_check(name, heads_checked, generator=None, storage_aware=False):
    """storage_aware: the max-abs bounds apply to the error beyond each element's bf16 output
    rounding (half a bf16 ulp of the reference), for inputs whose outputs exceed 16 in magnitude,
    where that rounding alone is larger than the 3e-2 gradient bound."""
    cfg = get_config(name)
    if generator:
        cfg = cfg.with_(generator=generator)
    log(f"[parity] {name} bf16 N={cfg.seq_len} H={cfg.heads} d={cfg.head_dim} r={cfg.rank} k={cfg.topk} "
        f"inputs {cfg.generator}")
    inp = make_inputs(cfg, workers=8)
    sc = _scale(cfg.head_dim)
    # oracle indices for the checked heads; other heads get a seeded list
    hs = list(heads_checked)
    x = {k: widen(v[:, hs]) if v.ndim == 4 else widen(v[hs]) for k, v in inp.items()}
    scores_o, qlr_o, klr_o = O.predict(x["q"], x["k"], x["wq"], x["wk"], cfg.q_block, cfg.kv_block, sc, "bf16")
    idx_o = O.select_topk(scores_o, cfg.topk)
    idx_fed = seeded_idx(7, (cfg.batch, cfg.heads), cfg.nqb, cfg.nkb, cfg.topk)
    idx_fed[:, hs] = idx_o
    r = _run_gpu_path(cfg, inp, idx_fed=idx_fed)
    # projections: the GPU rounds an fp32 accumulation (the query side scaled by
    # pred_scale * log2(e) in fp32) to bf16, the oracle the exact scaled product; they may differ by
    # the fp32 summation error (<= d * 2^-24 * sum|x w|, scaled), the fp32 rounding of the scaling
    # and one bf16 ulp
    qg, kg = to_f64(r["qlr"][:, hs]), to_f64(r["klr"][:, hs])
    for got, ref, xs, ws, s_ in ((qg, qlr_o, x["q"], x["wq"], sc * O.LOG2E), (kg, klr_o, x["k"], x["wk"], 1.0)):
        mag = np.maximum(np.abs(got), np.abs(ref))
        bound = bf16_ulp(mag) + 2.0 ** -24 * mag + s_ * cfg.head_dim * 2.0 ** -24 * np.einsum(
            "bhnd,hdr->bhnr", np.abs(xs), np.abs(ws))
        assert np.all(np.abs(got - ref) <= bound * 1.0001)
        assert (got != ref).mean() < 1e-2, (got != ref).mean()
    # scores: against the oracle's score step fed with the GPU's own projections
    sg = to_f64(r["scores"][:, hs])
    for bi in range(cfg.batch):
        for j in range(len(hs)):
            ref = O.block_scores_head(qg[bi, j], kg[bi, j], cfg.q_block, cfg.kv_block, O.LN2)
            np.testing.assert_allclose(sg[bi, j], ref, rtol=2e-4, atol=2e-5)
    np.testing.assert_allclose(to_f64(r["scores"]).sum(-1), cfg.q_block, rtol=1e-4)
    cov = check_indices(r["idx"][:, hs].cpu().numpy(), scores_o, cfg.topk)
    log(f"[parity] {name} index coverage (rows under the exact rule) {cov:.3f}")
    # forward with the oracle's indices
    o_o, lse_o = O.sparse_attn_fwd(x["q"], x["k"], x["v"], idx_o, cfg.q_block, cfg.kv_block, sc)
    og = to_f64(r["o"][:, hs])

    def beyond_storage(got, ref):  # error left after each element's bf16 output rounding
        return np.maximum(np.abs(got - ref) - (0.5 * bf16_ulp(np.abs(ref)) if storage_aware else 0.0), 0.0).max()

    err, rl2 = beyond_storage(og, o_o), rel_l2(og, o_o)
    log(f"[parity] {name} fwd max-abs {np.abs(og - o_o).max():.3e} (beyond bf16 output rounding {err:.3e}) "
        f"rel-L2 {rl2:.3e}")
    assert err <= FWD_BF16_MAXABS and rl2 <= FWD_BF16_RELL2
    assert np.abs(to_f64(r["lse"][:, hs]) - lse_o).max() <= 1e-2
    # backward
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], idx_o, cfg.q_block, cfg.kv_block, sc)
    for nm, got, ref in zip(("dq", "dk", "dv"), r["grads"], g_o):
        gg = to_f64(got[:, hs])
        e = beyond_storage(gg, ref)
        log(f"[parity] {name} {nm} max-abs {np.abs(gg - ref).max():.3e} (beyond bf16 output rounding {e:.3e}) "
            f"max|ref| {np.abs(ref).max():.1f} rel-L2 {rel_l2(gg, ref):.3e}")
        assert e <= GRAD_BF16_MAXABS and rel_l2(gg, ref) <= FWD_BF16_RELL2
    return cfg, inp, r, idx_fed


def test_c2_bf16_all_heads():
    cfg, inp, r, idx_fed = _bf16_config_check("C2", range(12))
    # determinism: a second run is bitwise identical
    r2 = _run_gpu_path(cfg, inp, idx_fed=idx_fed)
    for key in ("scores", "idx", "o", "lse"):
        assert torch.equal(r[key], r2[key]), key
    for a, b in zip(r["grads"], r2["grads"]):
        assert torch.equal(a, b)


def test_c3_bf16_sampled_heads():
    _bf16_config_check("C3", [0, 23])


def test_c3_g2_inputs():
    # 3D-cube token order with smooth Q and K fields: sharper, spatially coherent attention (more
    # rows under the exact index rule, and more rescaling in the forward's online softmax).
    # Gradients reach ~24 here, where half a bf16 ulp (0.0625) exceeds the 3e-2 bound by itself.
    _bf16_config_check("C3", [0, 11], generator="g2", storage_aware=True)


def test_o_residual_and_backward_without_it():
    # Asked for O's residual, the forward takes P V with P in fp16 (2^-11 relative instead of
    # bf16's 2^-8) and returns o_lo: o + o_lo is at least 4x closer to the oracle's O than the
    # plain forward's o.  The two forwards share the softmax statistics (lse is
    # identical), so the two backwards differ only through D = rowsum(dO * O):
    # dD_i = sum_c dO_ic ((o + o_lo) - o_plain)_ic.  dV does not depend on D, and since the sparse
    # softmax row P_i sums to 1, dQ moves by at most sm_scale * |dD_i| * max_{j selected} |K_jc|,
    # plus what each run's fp16 rounding of dS (relative 2^-11) can contribute,
    # 2 * 2^-11 * sm_scale * sum_j |dS_ij| |K_jc|, plus one bf16 ulp of each stored result.
    cfg = get_config("C2").with_(heads=4)
    log("[parity] O residual and backward without it (C2, 4 heads)")
    inp = make_inputs(cfg)
    x = {k: widen(v) for k, v in inp.items()}
    sc = _scale(cfg.head_dim)
    scores_o, _, _ = O.predict(x["q"], x["k"], x["wq"], x["wk"], cfg.q_block, cfg.kv_block, sc, "bf16")
    idx_o = O.select_topk(scores_o, cfg.topk)
    r = _run_gpu_path(cfg, inp, idx_fed=idx_o, residual=True)
    n = _run_gpu_path(cfg, inp, idx_fed=idx_o, residual=False)
    assert torch.equal(r["lse"], n["lse"])
    o_o, lse_o = O.sparse_attn_fwd(x["q"], x["k"], x["v"], idx_o, cfg.q_block, cfg.kv_block, sc)
    o_hi, o_lo, o_nr = to_f64(r["o"]), to_f64(r["o_lo"]), to_f64(n["o"])
    assert np.all(np.abs(o_lo) <= 0.5 * bf16_ulp(np.abs(o_hi)) * 1.0001)
    e_plain, e_full = np.abs(o_nr - o_o).max(), np.abs(o_hi + o_lo - o_o).max()
    log(f"[parity] O max-abs error: plain forward {e_plain:.3e}, o + o_lo {e_full:.3e}")
    assert e_full < 0.25 * e_plain
    assert np.abs(o_hi - o_o).max() <= FWD_BF16_MAXABS
    assert torch.equal(r["grads"][2], n["grads"][2])  # dV
    dd = (x["do"] * (o_hi + o_lo - o_nr)).sum(-1)  # [B, H, N]
    kmax = np.zeros_like(x["q"])
    dsk = np.zeros_like(x["q"])  # sum_j |dS_ij| |K_jc| over the selected keys
    for h in range(cfg.heads):
        for qb in range(cfg.nqb):
            keys = O.selected_keys(idx_o[0, h, qb], cfg.kv_block)
            rows = slice(qb * cfg.q_block, (qb + 1) * cfg.q_block)
            kk = x["k"][0, h][keys]
            kmax[0, h, rows] = np.abs(kk).max(0)
            p = np.exp(sc * x["q"][0, h, rows] @ kk.T - lse_o[0, h, rows, None])
            dp = x["do"][0, h, rows] @ x["v"][0, h][keys].T
            dvec = (x["do"][0, h, rows] * o_o[0, h, rows]).sum(-1)
            dsk[0, h, rows] = np.abs(p * (dp - dvec[:, None])) @ np.abs(kk)
    a, b = to_f64(r["grads"][0]), to_f64(n["grads"][0])
    bound = (sc * (np.abs(dd)[..., None] + 1e-5) * kmax + 2 * 2.0 ** -11 * sc * dsk
             + bf16_ulp(np.maximum(np.abs(a), np.abs(b))))
    log(f"[parity] dQ with vs without o_lo: max |diff| {np.abs(a - b).max():.3e}, min slack {(bound - np.abs(a - b)).min():.3e}")
    assert np.all(np.abs(a - b) <= bound)


# ------------------------------------------------------------------ small shapes: batch > 1, every instance, k = all


@pytest.mark.parametrize("d,bq,r", [(64, 64, 16), (64, 128, 32), (128, 64, 16), (128, 128, 32)])
def test_bf16_instances_batch2(d, bq, r):
    cfg = get_config("C2").with_(batch=2, heads=3, latent=(4, 16, 16), head_dim=d, rank=r, q_block=bq, topk=3)
    log(f"[parity] instance d={d} Bq={bq} r={r} B=2")
    inp = make_inputs(cfg)
    sc = _scale(d)
    x = {k: widen(v) for k, v in inp.items()}
    scores_o, _, _ = O.predict(x["q"], x["k"], x["wq"], x["wk"], bq, 64, sc, "bf16")
    idx_o = O.select_topk(scores_o, cfg.topk)
    rr = _run_gpu_path(cfg, inp, idx_fed=idx_o)
    check_indices(rr["idx"].cpu().numpy(), scores_o, cfg.topk)
    o_o, _ = O.sparse_attn_fwd(x["q"], x["k"], x["v"], idx_o, bq, 64, sc)
    og = to_f64(rr["o"])
    assert np.abs(og - o_o).max() <= FWD_BF16_MAXABS and rel_l2(og, o_o) <= FWD_BF16_RELL2
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], idx_o, bq, 64, sc)
    for got, ref in zip(rr["grads"], g_o):
        assert np.abs(to_f64(got) - ref).max() <= GRAD_BF16_MAXABS


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_all_blocks_selected_is_dense_attention(dtype):
    # k = N/Bk: the sparse kernels must reproduce dense attention (torch SDPA in fp32 on the CPU)
    cfg = get_config("C2").with_(heads=2, latent=(2, 16, 16), head_dim=64, rank=16, q_block=64, topk=8, dtype=dtype)
    log(f"[parity] dense special case {dtype}")
    inp = make_inputs(cfg)
    x = {k: widen(v) for k, v in inp.items()}
    idx = np.tile(np.arange(8, dtype=np.int32), (1, 2, 8, 1))
    rr = _run_gpu_path(cfg, inp, idx_fed=idx)
    assert np.array_equal(rr["idx"].cpu().numpy(), idx)  # k = nkb selects every block
    ref = torch.nn.functional.scaled_dot_product_attention(*(torch.from_numpy(x[n]).float() for n in ("q", "k", "v")))
    err = np.abs(to_f64(rr["o"]) - ref.double().numpy()).max()
    assert err <= (FWD_BF16_MAXABS if dtype == "bf16" else 1e-5), err


def test_single_block_and_unselected_blocks_get_zero_gradient():
    cfg = get_config("C2").with_(heads=1, latent=(2, 16, 16), head_dim=128, rank=32, q_block=128, topk=1)
    inp = make_inputs(cfg)
    x = {k: widen(v) for k, v in inp.items()}
    idx = np.full((1, 1, 4, 1), 3, dtype=np.int32)  # every query block picks KV block 3 only
    rr = _run_gpu_path(cfg, inp, idx_fed=idx)
    sc = _scale(128)
    o_o, _ = O.sparse_attn_fwd(x["q"], x["k"], x["v"], idx, 128, 64, sc)
    assert np.abs(to_f64(rr["o"]) - o_o).max() <= FWD_BF16_MAXABS
    dq, dk, dv = (to_f64(g) for g in rr["grads"])
    assert np.all(dk[0, 0, :192] == 0) and np.all(dv[0, 0, :192] == 0) and np.all(dk[0, 0, 256:] == 0)
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], idx, 128, 64, sc)
    for got, ref in zip((dq, dk, dv), g_o):
        assert np.abs(got - ref).max() <= GRAD_BF16_MAXABS


# ------------------------------------------------------------------ full-size configs, sampled outputs


@pytest.mark.parametrize("name", ["C4", "C4b", "C5", "NMAX", "C4-G2"])
def test_full_size_sampled(name):
    # NMAX: the largest sequence the library takes, N/Bk = 4096 KV blocks (N = 262144, a 64^3
    # latent), at C5's head shape and 10 % density, two heads.  C4-G2: C4 on the 3D-cube inputs
    # with smooth Q and K fields (larger gradients: bounds beyond the bf16 output rounding)
    if name == "NMAX":
        cfg = get_config("C5").with_(latent=(64, 64, 64), heads=2, topk=410)
    elif name == "C4-G2":
        cfg = get_config("C4").with_(generator="g2", heads=8)
    else:
        cfg = get_config(name)
    slack = (lambda ref: 0.5 * bf16_ulp(np.abs(ref))) if name == "C4-G2" else (lambda ref: 0.0)
    log(f"[parity] {name} full size N={cfg.seq_len} H={cfg.heads} k={cfg.topk}: generating inputs")
    inp = make_inputs(cfg, workers=16)
    sc = _scale(cfg.head_dim)
    idx_fed = seeded_idx(11, (cfg.batch, cfg.heads), cfg.nqb, cfg.nkb, cfg.topk)
    log(f"[parity] {name} running the GPU path")
    r = _run_gpu_path(cfg, inp, idx_fed=idx_fed)
    # properties over every row
    s_all = r["scores"]
    assert torch.isfinite(s_all).all()
    np.testing.assert_allclose(s_all.sum(-1).double().cpu().numpy(), cfg.q_block, rtol=2e-4)
    idx_all = r["idx"].cpu().numpy()
    assert np.all(np.diff(idx_all, axis=-1) > 0) and idx_all.min() >= 0 and idx_all.max() < cfg.nkb
    assert torch.isfinite(r["o"].float()).all()
    rng = np.random.default_rng(5)
    covered = []
    for h in (0, cfg.heads - 1):
        xq, xk, xv, xdo = (widen(inp[n][0, h]) for n in ("q", "k", "v", "do"))
        qlr_o = O.project_query(xq, widen(inp["wq"][h]), sc, "bf16")
        klr_o = O.project(xk, widen(inp["wk"][h]), "bf16")
        qg, kg = to_f64(r["qlr"][0, h]), to_f64(r["klr"][0, h])
        sg = to_f64(r["scores"][0, h])
        # the predictor's score rows element by element (the oracle fed the GPU's own projections,
        # as at the small sizes) and the selection of 16 sampled query blocks against the oracle
        for qb in rng.choice(cfg.nqb, size=16, replace=False):
            rows = slice(qb * cfg.q_block, (qb + 1) * cfg.q_block)
            ref = O.block_scores_qblock(qg[rows], kg, cfg.kv_block, O.LN2)
            np.testing.assert_allclose(sg[qb], ref, rtol=2e-4, atol=2e-5, err_msg=f"h={h} qb={qb}")
            s_o = O.block_scores_qblock(qlr_o[rows], klr_o, cfg.kv_block, O.LN2)
            covered.append(check_indices(idx_all[0, h, qb][None], s_o[None], cfg.topk))
        for qb in rng.choice(cfg.nqb, size=3, replace=False):
            rows = slice(qb * cfg.q_block, (qb + 1) * cfg.q_block)
            o_o, lse_o = O.attn_fwd_qblock(xq[rows], xk, xv, idx_fed[0, h, qb], cfg.kv_block, sc)
            og = to_f64(r["o"][0, h, rows])
            assert (np.abs(og - o_o) - slack(o_o)).max() <= FWD_BF16_MAXABS and rel_l2(og, o_o) <= FWD_BF16_RELL2
            assert np.abs(to_f64(r["lse"][0, h, rows]) - lse_o).max() <= 1e-2
            dq_o, _, _, _ = O.attn_bwd_qblock(xq[rows], xk, xv, xdo[rows], idx_fed[0, h, qb], cfg.kv_block, sc)
            assert (np.abs(to_f64(r["grads"][0][0, h, rows]) - dq_o) - slack(dq_o)).max() <= GRAD_BF16_MAXABS
            log(f"[parity] {name} h={h} qb={qb} forward and dQ ok")
        kbs = rng.choice(cfg.nkb, size=2, replace=False)
        for kb in kbs:
            dk_o, dv_o = O.attn_bwd_kvblock(xq, xk, xv, xdo, idx_fed[0, h], kb, cfg.q_block, cfg.kv_block, sc)
            keys = slice(kb * cfg.kv_block, (kb + 1) * cfg.kv_block)
            assert (np.abs(to_f64(r["grads"][1][0, h, keys]) - dk_o) - slack(dk_o)).max() <= GRAD_BF16_MAXABS
            assert (np.abs(to_f64(r["grads"][2][0, h, keys]) - dv_o) - slack(dv_o)).max() <= GRAD_BF16_MAXABS
            log(f"[parity] {name} h={h} kb={kb} dK/dV ok")
    cov = float(np.mean(covered))
    log(f"[parity] {name} index coverage: {len(covered)} sampled query blocks, {cov:.3f} under the exact rule")
    if name == "C4-G2":  # the 3D-cube inputs concentrate each query block's mass: the exact rule applies
        assert cov > 0


@pytest.mark.parametrize("r,bq", [(32, 128), (16, 64)])
def test_predictor_slots_running_several_items_with_exact_items_between(r, bq):
    # The score sweep runs persistent workgroups ("slots", 4 per compute unit), each taking items
    # of 256 query rows in turn; a fast item's masses are finalised during the slot's next sweep
    # and the slot's last item at its end, while an exact-path item is finalised at once.  540
    # heads of N = 1024 make 2160 items, so every slot runs two or three, and every third head
    # (overflowing block masses) or ninth (vanishing ones) takes the exact path between fast
    # items.  With W = [I; 0] the projections are the first r columns of Q and K; every head is
    # compared with the oracle on the GPU's own projections.
    heads, n, d, bk = 540, 1024, 64, 64
    rng = np.random.default_rng(37)
    q = rng.standard_normal((1, heads, n, d)).astype(np.float32)
    k = rng.standard_normal((1, heads, n, d)).astype(np.float32)
    over = [h for h in range(heads) if h % 3 == 1]
    tiny = [h for h in range(heads) if h % 9 == 5]
    q[0, over + tiny, :, :r] = 1.0
    big = 768.0 / r  # logits of ~138 (log2) on block 5: 2^138 overflows fp32
    k[0, over, 0:64, :r] = 0.0
    k[0, over, 5 * 64:6 * 64, :r] = big
    k[0, tiny, :, :r] = -big - np.abs(k[0, tiny, :, :r]) * 8
    k[0, tiny, 5 * 64:6 * 64, :r] = -big
    w = np.zeros((heads, d, r), np.float32)
    w[:, :r, :r] = np.eye(r)
    from workloads.generator import bf16_bits_from_f32
    t = {nm: to_dev(bf16_bits_from_f32(a)) for nm, a in (("q", q), ("k", k), ("w", w))}
    scores, qlr, klr = dsv.predict(t["q"], t["k"], t["w"], t["w"], q_block=bq, kv_block=bk, return_projections=True)
    torch.cuda.synchronize()
    sg, ql, kl = to_f64(scores)[0], to_f64(qlr)[0], to_f64(klr)[0]
    assert np.isfinite(sg).all()
    for h in range(heads):
        ref = O.block_scores_head(ql[h], kl[h], bq, bk, O.LN2)
        np.testing.assert_allclose(sg[h], ref, rtol=2e-4, atol=2e-5, err_msg=f"head {h}")
    assert np.all(sg[over, :, 5] > 0.99 * bq) and np.all(sg[tiny, :, 5] > 0.99 * bq)
    log(f"[parity] predictor r={r} bq={bq}: {heads} heads, {len(over) + len(tiny)} on the exact path, all match")


@pytest.mark.parametrize("n,heads,r,bq,check_every", [(256, 2100, 32, 128, 1), (4352, 130, 16, 64, 6),
                                                       (20480, 26, 32, 128, 5)])
def test_predictor_deferred_finalisation_at_edge_sizes(n, heads, r, bq, check_every):
    # Enough score items (heads * N / 256) that every persistent slot runs two or more, at the
    # edges of the deferred finalisation: N = 256 has 4 KV blocks (one chunk of 64, mostly past
    # the end) and more finalisation steps than sweep trips; N = 4352 has 68 KV blocks, so the
    # second chunk holds 4; N = 20480 has 320 KV blocks, five chunks, so wave 0 finalises two
    # (chunks 0 and 4), as every wave does at the full sizes.  Projections as in the test above
    # (W = [I; 0]).
    d, bk = 64, 64
    rng = np.random.default_rng(41)
    q = rng.standard_normal((1, heads, n, d)).astype(np.float32)
    k = rng.standard_normal((1, heads, n, d)).astype(np.float32)
    w = np.zeros((heads, d, r), np.float32)
    w[:, :r, :r] = np.eye(r)
    from workloads.generator import bf16_bits_from_f32
    t = {nm: to_dev(bf16_bits_from_f32(a)) for nm, a in (("q", q), ("k", k), ("w", w))}
    scores, qlr, klr = dsv.predict(t["q"], t["k"], t["w"], t["w"], q_block=bq, kv_block=bk, return_projections=True)
    torch.cuda.synchronize()
    sg, ql, kl = to_f64(scores)[0], to_f64(qlr)[0], to_f64(klr)[0]
    assert np.isfinite(sg).all()
    np.testing.assert_allclose(sg.sum(axis=-1), bq, rtol=1e-5)  # every row's masses sum to 1
    for h in range(0, heads, check_every):
        ref = O.block_scores_head(ql[h], kl[h], bq, bk, O.LN2)
        np.testing.assert_allclose(sg[h], ref, rtol=2e-4, atol=2e-5, err_msg=f"head {h}")
    log(f"[parity] predictor N={n} heads={heads} r={r} bq={bq}: every {check_every}th head matches")


@pytest.mark.parametrize("case", ["overflow", "tiny"])
def test_predictor_extreme_logits_use_the_exact_fallback(case):
    # With W = [I; 0], Q_lr and K_lr are the first r columns of Q and K, and every logit is
    # pred_scale * 16 * q * k (q = 1).  The fast sweep sums 2^logit without a shift; it is redone
    # with a per-block maximum when a row's total mass leaves [2^-100, fp32 max]:
    #  * overflow: block 5's keys give logits ~138 (log2), 2^138 overflows;
    #  * tiny: every key gives a logit <= ~-138 (log2), the total falls below 2^-100.
    n, d, r, bq, bk = 1024, 64, 16, 64, 64
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, 1, n, d)).astype(np.float32) * 0.1
    k = rng.standard_normal((1, 1, n, d)).astype(np.float32) * 0.1
    q[..., :r] = 1.0
    if case == "overflow":
        k[0, 0, 0:64, :r] = 0.0
        k[0, 0, 5 * 64:6 * 64, :r] = 48.0
    else:
        k[0, 0, :, :r] = -48.0 - np.abs(k[0, 0, :, :r]) * 200
        k[0, 0, 5 * 64:6 * 64, :r] = -48.0
    w = np.zeros((1, d, r), np.float32)
    w[0, :r, :r] = np.eye(r)
    from workloads.generator import bf16_bits_from_f32
    t = {nm: to_dev(bf16_bits_from_f32(a)) for nm, a in (("q", q), ("k", k), ("w", w))}
    scores, qlr, klr = dsv.predict(t["q"], t["k"], t["w"], t["w"], q_block=bq, kv_block=bk, return_projections=True)
    torch.cuda.synchronize()
    sg = to_f64(scores)[0, 0]
    ref = O.block_scores_head(to_f64(qlr)[0, 0], to_f64(klr)[0, 0], bq, bk, O.LN2)  # qlr: the scaled Q~
    assert np.isfinite(sg).all()
    np.testing.assert_allclose(sg, ref, rtol=2e-4, atol=2e-5)
    assert np.all(sg[:, 5] > 0.99 * bq)  # block 5 takes essentially all the mass


@pytest.mark.parametrize("r,bq", [(32, 128), (16, 64)])
def test_predictor_scores_do_not_depend_on_the_heads_sharing_a_call(r, bq):
    # The score sweep's persistent workgroups take items (256 query rows of one head) in turn.  A
    # workgroup finalises an item during its next item's sweep, or after its loop when the item was
    # its last; which items come last depends on the grid, the call's head count and the device.
    # Both finalisations must take the same arithmetic in the same order, so that a head's scores,
    # and with them its selection, are bit-identical whether it is predicted with all heads (2304
    # items: on a 256-CU device every workgroup runs two or three), in groups of 8 heads (128
    # items, each the last of its workgroup) or alone.
    heads, n, d, bk, topk = 144, 4096, 64, 64, 7
    rng = np.random.default_rng(53)
    from workloads.generator import bf16_bits_from_f32
    q = bf16_bits_from_f32(rng.standard_normal((1, heads, n, d)).astype(np.float32))
    k = bf16_bits_from_f32(rng.standard_normal((1, heads, n, d)).astype(np.float32))
    w = bf16_bits_from_f32((rng.standard_normal((2, heads, d, r)) / np.sqrt(d)).astype(np.float32))
    t = {nm: to_dev(a) for nm, a in (("q", q), ("k", k), ("wq", w[0]), ("wk", w[1]))}
    kw = dict(q_block=bq, kv_block=bk)
    full = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], **kw)
    grouped = torch.empty_like(full)
    for h0 in range(0, heads, 8):
        sl = slice(h0, h0 + 8)
        dsv.predict(t["q"][:, sl], t["k"][:, sl], t["wq"][sl], t["wk"][sl], out=grouped[:, sl], **kw)
    alone = [dsv.predict(t["q"][:, h:h + 1], t["k"][:, h:h + 1], t["wq"][h:h + 1], t["wk"][h:h + 1], **kw)
             for h in (0, heads - 1)]
    idx_full = dsv.select_topk(full, topk, **kw)
    idx_grouped = dsv.select_topk(grouped, topk, **kw)
    torch.cuda.synchronize()
    assert torch.equal(full, grouped)
    assert torch.equal(full[:, :1], alone[0]) and torch.equal(full[:, -1:], alone[1])
    assert torch.equal(idx_full, idx_grouped)
    np.testing.assert_allclose(to_f64(full).sum(axis=-1), bq, rtol=1e-5)
    log(f"[parity] predictor r={r} bq={bq}: {heads} heads bit-equal alone, in groups of 8 and all at once")


def test_attention_results_do_not_depend_on_the_heads_sharing_a_call():
    # Forward and backward on all heads at once, and head group by head group (4 calls of 3
    # heads), on the same lists: every output bit-equal.  Each head's fp16 scales come from that
    # head's own maxima, and no workgroup mixes heads.
    cfg = get_config("C2")
    inp = make_inputs(cfg, with_grad=True)
    t = {k: to_dev(v) for k, v in inp.items()}
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block)
    idx_d = to_dev(seeded_idx(11, (cfg.batch, cfg.heads), cfg.nqb, cfg.nkb, cfg.topk))
    o, lse, o_lo = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx_d, residual=True, **kw)
    full = (o, lse) + tuple(dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, idx_d, o_lo=o_lo, **kw))
    parts = [torch.empty_like(x) for x in full]
    for h0 in range(0, cfg.heads, 3):
        sl = slice(h0, h0 + 3)
        q, k, v, do = (t[n][:, sl] for n in ("q", "k", "v", "do"))
        og, lg, olg = dsv.sparse_attn_fwd(q, k, v, idx_d[:, sl], residual=True, **kw)
        grads = dsv.sparse_attn_bwd(q, k, v, og, do, lg, idx_d[:, sl], o_lo=olg, **kw)
        for dst, src in zip(parts, (og, lg) + tuple(grads)):
            dst[:, sl] = src
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), full, parts):
        assert torch.equal(a, b), name
    log(f"[parity] C2 attention: {cfg.heads} heads bit-equal at once and in groups of 3")


def test_autograd_function_gradients_match_the_oracle():
    # DSVAttention.apply: predict -> select -> training forward, and the sparse backward through
    # autograd.  The q, k, v gradients must match the oracle's backward on the GPU-chosen indices
    # within the gradient bound; the predictor weights get no gradient, and the index list is not
    # differentiable.
    cfg = get_config("C2").with_(heads=3)
    log("[parity] autograd Function (C2, 3 heads)")
    inp = make_inputs(cfg)
    t = {k: to_dev(v) for k, v in inp.items()}
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    wq, wk = t["wq"].clone().requires_grad_(True), t["wk"].clone().requires_grad_(True)
    o, idx = dsv.DSVAttention.apply(q, k, v, wq, wk, cfg.q_block, cfg.kv_block, cfg.topk)
    assert not idx.requires_grad and idx.dtype == torch.int32
    o.backward(t["do"])
    torch.cuda.synchronize()
    assert wq.grad is None and wk.grad is None
    x = {n: widen(a) for n, a in inp.items()}
    sc = _scale(cfg.head_dim)
    gi = idx.cpu().numpy()
    s_o, _, _ = O.predict(x["q"], x["k"], x["wq"], x["wk"], cfg.q_block, cfg.kv_block, sc, "bf16")
    cov = check_indices(gi, s_o, cfg.topk)
    o_o, _ = O.sparse_attn_fwd(x["q"], x["k"], x["v"], gi, cfg.q_block, cfg.kv_block, sc)
    assert np.abs(to_f64(o) - o_o).max() <= FWD_BF16_MAXABS and rel_l2(to_f64(o), o_o) <= FWD_BF16_RELL2
    g_o = O.sparse_attn_bwd(x["q"], x["k"], x["v"], x["do"], gi, cfg.q_block, cfg.kv_block, sc)
    for nm, got, ref in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), g_o):
        err = np.abs(to_f64(got) - ref).max()
        log(f"[parity] autograd {nm} max-abs {err:.3e}")
        assert got.dtype == torch.bfloat16 and err <= GRAD_BF16_MAXABS
    log(f"[parity] autograd: index coverage {cov:.3f}")
