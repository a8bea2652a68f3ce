"""Seeded synthetic video-token tensors for the DSV attention workloads.

What the inputs stand in for: the DSV explainer pages (gist.science/de/paper/
2502.07590, "Technische Zusammenfassung" §1 and §3; Spanish version §1) state
that attention in video DiTs is dominated by a small, dynamic, non-local set
of critical key-value pairs, and that tokens adjacent in the 3D latent grid
tend to share them (§2.B, query grouping).  No activations of a trained model
are available, so the recipe below builds tensors with that structure from
seeded Gaussian noise:

* ``plain``: Q, K, V, dO ~ N(0, 1) i.i.d.; predictor weights ~ N(0, 1/d).
* ``g1``: as ``plain``, plus a spatially smooth per-head field F_K added to K
  (K = noise + alpha * F_K, alpha = 2.5).  F_K is white noise on the
  (T, H, W, d) grid, blurred with a periodic separable Gaussian of sigma = 2
  cells along t, y and x (taps truncated at |offset| <= 8), then standardised
  per channel.  Tokens are in raster order n = (t*H + y)*W + x.
* ``g2``: ``g1`` plus an independent smooth field on Q (Q += alpha * F_Q), with
  tokens reordered into 4x4x4 cubes (cubes in raster order, raster order inside
  a cube), so that a 64-token block is a 3D-compact cube.

Every draw comes from ``numpy.random.default_rng([seed, tensor_id, b, h])`` as
float32 standard normals; generation is per (b, h), so a subset of heads can be
regenerated bit-identically.  bf16 storage is produced by round-to-nearest-even
from the float32 draws.  This module contains no attention arithmetic.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np

from .configs import Config

# tensor ids of the seeded streams
TID_Q, TID_K, TID_V, TID_FK, TID_FQ, TID_WQ, TID_WK, TID_DO = range(8)

SIGMA = 2.0
TRUNC = 8


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, tid: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid, b, h])


def _normal(seed, tid, b, h, shape) -> np.ndarray:
    return _rng(seed, tid, b, h).standard_normal(size=shape, dtype=np.float32)


def _periodic_taps(length: int) -> np.ndarray:
    """Gaussian taps (sigma=SIGMA, |offset|<=TRUNC), normalised, folded onto a ring of `length`."""
    taps = np.zeros(length, dtype=np.float64)
    offs = np.arange(-TRUNC, TRUNC + 1)
    g = np.exp(-(offs.astype(np.float64) ** 2) / (2.0 * SIGMA * SIGMA))
    g /= g.sum()
    for o, w in zip(offs, g):
        taps[o % length] += w
    return taps


def _blur_axis(x: np.ndarray, axis: int) -> np.ndarray:
    n = x.shape[axis]
    if n == 1:
        return x
    spec = np.fft.rfft(_periodic_taps(n)).real.astype(np.float32)  # the taps are even: real spectrum
    shape = [1] * x.ndim
    shape[axis] = spec.shape[0]
    return np.fft.irfft(np.fft.rfft(x, axis=axis) * spec.reshape(shape), n=n, axis=axis).astype(np.float32)


def smooth_field(seed: int, tid: int, b: int, h: int, latent, d: int) -> np.ndarray:
    """Standardised, Gaussian-blurred noise on the (T, H, W, d) grid, float32 [T, H, W, d].

    The blur runs in float32 (single-precision FFTs); the per-channel mean and
    standard deviation are accumulated in float64.
    """
    t, hh, w = latent
    f = _normal(seed, tid, b, h, (t, hh, w, d))
    for ax in range(3):
        f = _blur_axis(f, ax)
    mu = f.mean(axis=(0, 1, 2), keepdims=True, dtype=np.float64)
    sd = f.std(axis=(0, 1, 2), keepdims=True, dtype=np.float64)
    return ((f - mu) / np.where(sd > 0, sd, 1.0)).astype(np.float32)


def cube_order(latent) -> np.ndarray:
    """Permutation perm such that token i of the reordered sequence is raster token perm[i].

    Tokens are grouped into 4x4x4 cubes (cubes in raster order of their corner,
    raster order inside a cube).  Each axis length must be a multiple of 4.
    """
    t, hh, w = latent
    if t % 4 or hh % 4 or w % 4:
        raise ValueError("cube order needs every latent axis to be a multiple of 4")
    ct, cy, cx = np.meshgrid(np.arange(t // 4), np.arange(hh // 4), np.arange(w // 4), indexing="ij")
    it, iy, ix = np.meshgrid(np.arange(4), np.arange(4), np.arange(4), indexing="ij")
    tt = (ct.reshape(-1, 1) * 4 + it.reshape(1, -1)).reshape(-1)
    yy = (cy.reshape(-1, 1) * 4 + iy.reshape(1, -1)).reshape(-1)
    xx = (cx.reshape(-1, 1) * 4 + ix.reshape(1, -1)).reshape(-1)
    return ((tt * hh + yy) * w + xx).astype(np.int64)


def _to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(x32)
    raise ValueError(dtype)


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 values of a storage array (float32, or uint16 bf16 patterns)."""
    if x.dtype == np.uint16:
        return f32_from_bf16_bits(x).astype(np.float64)
    return x.astype(np.float64)


def make_head(cfg: Config, b: int, h: int, with_grad: bool = True) -> Dict[str, np.ndarray]:
    """Float32 values (before storage rounding) of one (b, h) head: q, k, v, do [N, d]; wq, wk [d, r]."""
    n, d, r, s = cfg.seq_len, cfg.head_dim, cfg.rank, cfg.seed
    q = _normal(s, TID_Q, b, h, (n, d))
    k = _normal(s, TID_K, b, h, (n, d))
    v = _normal(s, TID_V, b, h, (n, d))
    if cfg.generator in ("g1", "g2"):
        fk = smooth_field(s, TID_FK, b, h, cfg.latent, d).reshape(n, d)
        k = k + np.float32(cfg.bias_alpha) * fk
    if cfg.generator == "g2":
        fq = smooth_field(s, TID_FQ, b, h, cfg.latent, d).reshape(n, d)
        q = q + np.float32(cfg.bias_alpha) * fq
        perm = cube_order(cfg.latent)
        q, k, v = q[perm], k[perm], v[perm]
    # predictor weights are per head (b-independent): seeded with b = 0
    wq = (_normal(s, TID_WQ, 0, h, (d, r)).astype(np.float64) / math.sqrt(d)).astype(np.float32)
    wk = (_normal(s, TID_WK, 0, h, (d, r)).astype(np.float64) / math.sqrt(d)).astype(np.float32)
    out = {"q": q, "k": k, "v": v, "wq": wq, "wk": wk}
    if with_grad:
        out["do"] = _normal(s, TID_DO, b, h, (n, d))
    return out


def _head_job(args):
    cfg, b, h, with_grad = args
    t = make_head(cfg, b, h, with_grad)
    return {nm: _to_storage(x, cfg.dtype) for nm, x in t.items()}


def make_inputs(cfg: Config, heads: Optional[Iterable[int]] = None, with_grad: Optional[bool] = None,
                batches: Optional[Iterable[int]] = None, workers: int = 1) -> Dict[str, np.ndarray]:
    """Storage arrays for the selected heads (default: all).

    Returns q, k, v (and do) as [B', H', N, d] and wq, wk as [H', d, r], in the
    config's storage dtype: float32 arrays for "f32", uint16 bf16 bit patterns
    for "bf16".  Use :func:`widen` for their exact float64 values.  ``workers``
    > 1 generates heads on that many threads (same values; NumPy's generators
    and FFTs release the GIL).  Threads rather than forked processes, so that
    generation is safe inside processes that already run threads of their own
    (profilers, GPU runtimes).
    """
    if with_grad is None:
        with_grad = cfg.backward
    hs = list(range(cfg.heads)) if heads is None else list(heads)
    bs = list(range(cfg.batch)) if batches is None else list(batches)
    n, d, r = cfg.seq_len, cfg.head_dim, cfg.rank
    sdt = np.float32 if cfg.dtype == "f32" else np.uint16
    names = ["q", "k", "v"] + (["do"] if with_grad else [])
    out = {nm: np.empty((len(bs), len(hs), n, d), dtype=sdt) for nm in names}
    out["wq"] = np.empty((len(hs), d, r), dtype=sdt)
    out["wk"] = np.empty((len(hs), d, r), dtype=sdt)
    jobs = [(cfg, b, h, with_grad) for b in bs for h in hs]
    if workers > 1 and len(jobs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(workers, len(jobs))) as pool:
            results = list(pool.map(_head_job, jobs))
    else:
        results = map(_head_job, jobs)
    for j, t in enumerate(results):
        bi, hi = divmod(j, len(hs))
        for nm in names:
            out[nm][bi, hi] = t[nm]
        if bi == 0:
            out["wq"][hi] = t["wq"]
            out["wk"][hi] = t["wk"]
    return out
