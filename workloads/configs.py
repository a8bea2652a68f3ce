"""Problem sizes of the synthetic video-DiT attention workloads.

The DSV explainer pages (gist.science/de|es/paper/2502.07590, "Technical
summary" §1 and §4) describe video DiTs whose 3D self-attention runs over
T x H x W latent tokens, up to hundreds of thousands of tokens.  The pages give
no block sizes, ranks or k; the sizes below are the synthetic workloads this
library is measured and checked on, from a tiny fp32 case to a 131072-token
long-video layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    heads: int
    latent: Tuple[int, int, int]  # (T, H, W) latent grid; N = T*H*W tokens
    head_dim: int
    rank: int
    q_block: int
    kv_block: int
    topk: int
    dtype: str  # "f32" or "bf16"
    backward: bool
    generator: str  # "plain" (i.i.d. normal) or "g1" / "g2" (smooth bias on K)
    seed: int
    bias_alpha: float = 2.5
    note: str = field(default="", compare=False)

    @property
    def seq_len(self) -> int:
        t, h, w = self.latent
        return t * h * w

    @property
    def nqb(self) -> int:
        return self.seq_len // self.q_block

    @property
    def nkb(self) -> int:
        return self.seq_len // self.kv_block

    def fwd_flops(self) -> float:
        """Algorithmic forward flops: two GEMMs (S=QK^T, O=PV) over the selected keys."""
        return 4.0 * self.batch * self.heads * self.seq_len * (self.topk * self.kv_block) * self.head_dim

    def bwd_flops(self) -> float:
        """Algorithmic backward flops: five GEMMs (S, dP, dV, dK, dQ) = 2.5x forward."""
        return 2.5 * self.fwd_flops()

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


def _c(name, b, h, latent, d, r, bq, bk, k, dtype, bwd, gen, seed, note=""):
    return Config(name, b, h, latent, d, r, bq, bk, k, dtype, bwd, gen, seed, note=note)


CONFIGS = {
    # Tiny fp32 forward-only case: the oracle finishes it in well under a second.
    "C1": _c("C1", 1, 2, (4, 16, 16), 64, 16, 64, 64, 2, "f32", False, "plain", 1001,
             "tiny fp32 forward, 16x16 blocks, top-2"),
    "C2": _c("C2", 1, 12, (8, 32, 32), 64, 16, 64, 64, 13, "bf16", True, "g1", 1002,
             "N=8192, 13 of 128 KV blocks"),
    "C3": _c("C3", 1, 24, (16, 32, 32), 128, 32, 64, 64, 26, "bf16", True, "g1", 1003,
             "N=16384, 26 of 256 KV blocks"),
    "C4": _c("C4", 1, 40, (16, 64, 64), 128, 32, 128, 64, 103, "bf16", True, "g1", 1004,
             "N=65536, 103 of 1024 KV blocks (10%)"),
    "C4b": _c("C4b", 1, 40, (16, 64, 64), 128, 32, 128, 64, 51, "bf16", True, "g1", 1004,
              "N=65536, 51 of 1024 KV blocks (5%)"),
    "C5": _c("C5", 1, 40, (32, 64, 64), 128, 32, 128, 64, 205, "bf16", True, "g1", 1005,
             "N=131072 long-video layer, 205 of 2048 KV blocks (10%)"),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]
