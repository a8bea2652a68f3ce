"""Index-rule coverage and captured attention mass of the synthetic workloads, from the CPU oracle.

For sampled query blocks of each config and input generator:
  * coverage: the fraction of query blocks whose oracle top-k gap s_(k) - s_(k+1) exceeds 1e-3,
    i.e. where the GPU's selection must equal the oracle's bit for bit (elsewhere any near-tie
    choice is valid), and the median gap;
  * the true softmax mass (sm_scale = 1/sqrt(d), over all N keys) that a query block's rows put
    on: each row's own best k blocks (an upper bound no shared list reaches), the query block's
    best k blocks by summed true mass (the best a shared top-k list can do), and the predicted
    top-k (the oracle's selection from the random-init predictor).
The pages' premise is that about 10 % of the KV blocks carry about 90 % of the attention score
(DSV explainer, German and Spanish pages, technical summary 2.A).

Usage: python -m tests.index_coverage [--out profiles/index_coverage.md] [--qblocks 16] [--heads 2]
"""
from __future__ import annotations

import argparse
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import dsv_oracle as O  # noqa: E402
from workloads import get_config, make_inputs  # noqa: E402
from workloads.generator import widen  # noqa: E402


def measure(name, gen, heads, nq, seed=0):
    cfg = get_config(name).with_(generator=gen)
    hs = sorted({0, cfg.heads - 1} if heads >= 2 else {0})
    inp = make_inputs(cfg, heads=hs, with_grad=False, workers=8)
    ps = ss = 1.0 / math.sqrt(cfg.head_dim)
    bq, bk, k = cfg.q_block, cfg.kv_block, cfg.topk
    rng = np.random.default_rng(seed)
    gaps, row_best, blk_best, pred = [], [], [], []
    for j, h in enumerate(hs):
        q, kk = widen(inp["q"][0, j]), widen(inp["k"][0, j])
        qt = O.project_query(q, widen(inp["wq"][j]), ps, cfg.dtype)
        kl = O.project(kk, widen(inp["wk"][j]), cfg.dtype)
        for qb in rng.choice(cfg.nqb, size=min(nq, cfg.nqb), replace=False):
            rows = slice(qb * bq, (qb + 1) * bq)
            s = O.block_scores_qblock(qt[rows], kl, bk, O.LN2)
            gaps.append(float(O.topk_gap(s[None], k)[0]))
            sel = O.select_topk_row(s, k)
            logits = ss * q[rows] @ kk.T
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            m = p.reshape(bq, cfg.nkb, bk).sum(axis=2)          # true mass per (row, KV block)
            row_best.append(float(np.sort(m, axis=1)[:, -k:].sum(axis=1).mean()))
            blk_best.append(float(np.sort(m.sum(axis=0))[-k:].sum() / bq))
            pred.append(float(m[:, sel].sum(axis=1).mean()))
    g = np.array(gaps)
    return dict(cfg=cfg, n=len(gaps), cov=float((g > 1e-3).mean()), med=float(np.median(g)),
                row_best=float(np.mean(row_best)), blk_best=float(np.mean(blk_best)), pred=float(np.mean(pred)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "index_coverage.md"))
    ap.add_argument("--qblocks", type=int, default=16, help="sampled query blocks per head")
    ap.add_argument("--heads", type=int, default=2, help="heads per config (the first and the last)")
    ap.add_argument("--configs", default="C2,C3,C4,C4b,C5")
    a = ap.parse_args()
    lines = ["# Index-rule coverage and captured attention mass (CPU oracle)", "",
             f"Command: `python -m tests.index_coverage --qblocks {a.qblocks} --heads {a.heads} "
             f"--configs {a.configs}`", "",
             f"{a.qblocks} sampled query blocks in each of the first and last head (seed 0). "
             "Coverage: query blocks whose oracle top-k gap exceeds 1e-3 (bit-exact index rule). "
             "True mass: the exact softmax mass (sm_scale = 1/sqrt(d), all N keys) a query block's rows "
             "put on the blocks named, averaged over rows. Predictor: random-init Wq, Wk.", "",
             "| Config | Generator | k / N/Bk | Query blocks | Coverage (gap > 1e-3) | Median gap | "
             "Per-row best k blocks | Best shared top-k | Predicted top-k |",
             "|---|---|---|---|---|---|---|---|---|"]
    for name in a.configs.split(","):
        for gen in ("g1", "g2"):
            t0 = time.perf_counter()
            r = measure(name, gen, a.heads, a.qblocks)
            c = r["cfg"]
            lines.append(f"| {name} | {gen.upper()} | {c.topk} / {c.nkb} | {r['n']} | {r['cov']:.3f} | {r['med']:.1e} | "
                         f"{r['row_best']:.3f} | {r['blk_best']:.3f} | {r['pred']:.3f} |")
            print(lines[-1], f"({time.perf_counter() - t0:.0f} s)", flush=True)
    os.makedirs(os.path.dirname(a.out), exist_ok=True)
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {a.out}")


if __name__ == "__main__":
    main()
