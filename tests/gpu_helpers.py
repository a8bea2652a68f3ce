"""Helpers shared by the GPU parity tests: moving storage arrays to the device,
bringing results back as exact float64, and the comparison criteria."""
import sys

import numpy as np
import torch

from oracle import dsv_oracle as O
from workloads.generator import widen

# Acceptance bars (from the project's stated criteria):
GAP = 1e-3            # indices must match bit-exactly where the oracle's s_(k) - s_(k+1) exceeds this
FWD_F32_MAXABS = 1e-5
FWD_BF16_MAXABS = 2e-2
FWD_BF16_RELL2 = 5e-3
GRAD_BF16_MAXABS = 3e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """Storage array -> device tensor (uint16 bit patterns become bfloat16)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> exact float64 numpy values."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def check_indices(gpu_idx: np.ndarray, oracle_scores: np.ndarray, k: int, gap_rule: float = GAP):
    """Index criterion.  Rows whose oracle gap s_(k) - s_(k+1) > gap_rule must match the
    oracle's selection exactly; every other row must be a valid near-tie choice:
    each selected block scores >= s_(k) - gap_rule and each dropped block <= s_(k+1) + gap_rule.
    Also checks every row is ascending and duplicate-free.  Returns the coverage
    (fraction of rows under the exact rule)."""
    GAP = gap_rule  # noqa: N806
    s = oracle_scores.reshape(-1, oracle_scores.shape[-1])
    g = gpu_idx.reshape(-1, gpu_idx.shape[-1]).astype(np.int64)
    assert np.all(np.diff(g, axis=1) > 0), "rows must be strictly ascending"
    assert g.min() >= 0 and g.max() < s.shape[1]
    want = O.select_topk(s, k)
    gap = O.topk_gap(s, k)
    exact = gap > GAP
    bad = np.nonzero(exact & np.any(g != want, axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows with gap > {GAP} differ, first {bad[:5]}"
    srt = -np.sort(-s, axis=1)
    sk = srt[:, k - 1]
    sk1 = srt[:, k] if k < s.shape[1] else np.full(s.shape[0], -np.inf)
    for r in np.nonzero(~exact)[0]:
        sel = np.zeros(s.shape[1], bool)
        sel[g[r]] = True
        assert s[r, sel].min() >= sk[r] - GAP, r
        if k < s.shape[1]:
            assert s[r, ~sel].max() <= sk1[r] + GAP, r
    return float(exact.mean())


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits; fixed 2^-133 below 2^-126)."""
    e = np.frexp(np.abs(x))[1]
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def seeded_idx(seed: int, shape_bh, nqb: int, nkb: int, k: int) -> np.ndarray:
    """Random ascending, duplicate-free block lists (an input, drawn from a seeded generator)."""
    rng = np.random.default_rng(seed)
    b, h = shape_bh
    out = np.empty((b, h, nqb, k), dtype=np.int32)
    for bi in range(b):
        for hi in range(h):
            for q in range(nqb):
                out[bi, hi, q] = np.sort(rng.choice(nkb, size=k, replace=False))
    return out
