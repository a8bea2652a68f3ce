"""MI355X (gfx950) DSV dynamic block-sparse attention.

A thin Python binding over the C ABI of ``libdsv.so`` (declared in
``include/dsv.h``).  It only marshals arguments: torch tensors provide device
memory and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is missing, or the
tensors are not on a GPU, the calls raise.

Entry points (same names as the C ABI):
  predict(q, k, wq, wk, ...)          -> block_scores [B, H, N/Bq, N/Bk] float32 (rep_row=...: one-row masses)
  predict_select_representative(q, k, wq, wk, topk, rep_row, ...) -> block_idx (fused predict + top-k)
  select_topk(block_scores, topk)     -> block_idx    [B, H, N/Bq, k]    int32
  select_mass(block_scores, tau, kmax) -> (block_idx [B, H, N/Bq, kmax] padded with -1, block_counts)
  sparse_attn_fwd(q, k, v, idx, ...)  -> (o, lse), or (o, lse, o_lo) with residual=True
  sparse_attn_bwd(q, k, v, o, do, lse, idx, ..., o_lo=None) -> (dq, dk, dv)
  block_recall(lse_selected, lse_all, q_block) -> recall [B, H, N/Bq] (true mass captured)
  head_density(block_counts, topk, ...) -> (density [B, H], dense flag [B, H])
  pack_kv(k, v, idx, qb_begin, qb_end, ...) -> (k_packed, v_packed, packed_blocks, packed_counts, packed_idx)
  pack_kv_noalloc(...)                 the same without a workspace (the library's own device array)
  peak_probe(kind)                     the rate this device sustains for one bounding operation
  DSVAttention.apply(q, k, v, wq, wk, q_block, kv_block, topk) -> (o, block_idx), differentiable in q, k, v
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsv.so")

DSV_F32, DSV_BF16 = 0, 1
STATUS = {0: "DSV_OK", 1: "DSV_ERR_INVALID_ARGUMENT", 2: "DSV_ERR_UNSUPPORTED", 3: "DSV_ERR_WORKSPACE_TOO_SMALL",
          4: "DSV_ERR_HIP"}

EXPORTED = ("dsv_predict_workspace_size", "dsv_predict", "dsv_predict_representative",
            "dsv_predict_select_representative", "dsv_select_topk",
            "dsv_select_mass", "dsv_head_density", "dsv_block_recall", "dsv_pack_kv_workspace_size", "dsv_pack_kv",
            "dsv_pack_kv_noalloc",
            "dsv_sparse_attn_fwd_workspace_size",
            "dsv_sparse_attn_fwd", "dsv_sparse_attn_bwd_workspace_size", "dsv_sparse_attn_bwd", "dsv_status_string",
            "dsv_last_error", "dsv_version", "dsv_timing_begin", "dsv_timing_end", "dsv_peak_probe_workspace_size",
            "dsv_peak_probe")


class Problem(ctypes.Structure):
    """Mirror of ``dsv_problem`` in include/dsv.h."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("q_block", ctypes.c_int32), ("kv_block", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("pred_scale", ctypes.c_float)]


class KernelStat(ctypes.Structure):
    """Mirror of ``dsv_kernel_stat`` in include/dsv.h."""
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double),
                ("min_ms", ctypes.c_float), ("max_ms", ctypes.c_float)]


class DSVError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsv.so (once) and declare the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m dynamic_sparse_attention_dsv_amd.build`")
    lib = ctypes.CDLL(path)
    P, V, S = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "dsv_predict_workspace_size": (S, [P]),
        "dsv_predict": (ctypes.c_int, [P, V, V, V, V, V, S, V, V]),
        "dsv_predict_representative": (ctypes.c_int, [P, V, V, V, V, ctypes.c_int32, V, S, V, V]),
        "dsv_predict_select_representative": (ctypes.c_int, [P, V, V, V, V, ctypes.c_int32, V, S, V, V]),
        "dsv_select_topk": (ctypes.c_int, [P, V, V, V]),
        "dsv_select_mass": (ctypes.c_int, [P, V, ctypes.c_float, V, V, V]),
        "dsv_block_recall": (ctypes.c_int, [P, V, V, V, V]),
        "dsv_head_density": (ctypes.c_int, [P, V, ctypes.c_float, V, V, V]),
        "dsv_pack_kv_workspace_size": (S, [P]),
        "dsv_pack_kv": (ctypes.c_int, [P, V, V, V, V, ctypes.c_int32, ctypes.c_int32, V, V, V, V, V, V, S, V]),
        "dsv_pack_kv_noalloc": (ctypes.c_int, [P, V, V, V, V, ctypes.c_int32, ctypes.c_int32, V, V, V, V, V, V]),
        "dsv_sparse_attn_fwd_workspace_size": (S, [P]),
        "dsv_sparse_attn_fwd": (ctypes.c_int, [P, V, V, V, V, V, V, V, V, V, S, V]),
        "dsv_sparse_attn_bwd_workspace_size": (S, [P]),
        "dsv_sparse_attn_bwd": (ctypes.c_int, [P, V, V, V, V, V, V, V, V, V, V, V, V, V, S, V]),
        "dsv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "dsv_last_error": (ctypes.c_char_p, []),
        "dsv_version": (ctypes.c_int32, []),
        "dsv_timing_begin": (ctypes.c_int, []),
        "dsv_timing_end": (ctypes.c_int32, [ctypes.POINTER(KernelStat), ctypes.c_int32]),
        "dsv_peak_probe_workspace_size": (S, [ctypes.c_int32]),
        "dsv_peak_probe": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, V, S, ctypes.POINTER(ctypes.c_double), V]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DSVError(status, where, load_library().dsv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSV_BF16
    if t.dtype == torch.float32:
        return DSV_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _dev(*ts: torch.Tensor) -> torch.device:
    ts = [t for t in ts if t is not None]
    dev = ts[0].device
    if dev.type != "cuda":
        raise RuntimeError("dsv kernels need GPU tensors (no CPU path exists)")
    for t in ts:
        if t.device != dev:
            raise RuntimeError("all tensors must be on the same device")
    return dev


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype) -> None:
    """Shape and dtype of a tensor the kernels will read or write: a mismatch would make them
    touch memory outside the allocation, so it is refused here, before any device work."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_counts(cnt: Optional[torch.Tensor], idx: torch.Tensor) -> None:
    if cnt is not None:
        _expect(cnt, "block_counts", idx.shape[:-1], torch.int32)


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def make_problem(q: torch.Tensor, *, q_block: int, kv_block: int, topk: int = 1, rank: int = 0,
                 sm_scale: Optional[float] = None, pred_scale: Optional[float] = None) -> Problem:
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    b, h, n, d = q.shape
    return Problem(b, h, n, d, q_block, kv_block, topk, rank, _dtype_code(q),
                   0.0 if sm_scale is None else float(sm_scale), 0.0 if pred_scale is None else float(pred_scale))


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _blocks(n: int, q_block: int, kv_block: int) -> Tuple[int, int]:
    if q_block < 1 or kv_block < 1 or n % q_block or n % kv_block:
        raise ValueError(f"N={n} must be a multiple of q_block={q_block} and kv_block={kv_block}")
    return n // q_block, n // kv_block


def _workspace(nbytes: int, dev: torch.device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def predict_workspace_size(prob: Problem) -> int:
    return int(load_library().dsv_predict_workspace_size(ctypes.byref(prob)))


def _predict_inputs(q, k, wq, wk):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    b, h, n, d = q.shape
    _expect(k, "k", q.shape, q.dtype)
    if wq.dim() != 3:
        raise ValueError("wq must be [H, d, r]")
    _expect(wq, "wq", (h, d, wq.shape[2]), q.dtype)
    _expect(wk, "wk", wq.shape, q.dtype)
    _contig(q)
    return b, h, n, d, wq.shape[2]


def _projections(ws, q, b, h, n, r):
    esz = q.element_size()
    lr = b * h * n * r * esz
    off_k = (lr + 255) // 256 * 256
    flat = ws.view(torch.uint8)
    return flat[:lr].view(q.dtype).view(b, h, n, r), flat[off_k:off_k + lr].view(q.dtype).view(b, h, n, r)


def predict(q, k, wq, wk, *, q_block: int, kv_block: int = 64, pred_scale: Optional[float] = None,
            rep_row: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
            return_projections: bool = False, out: Optional[torch.Tensor] = None):
    """Predicted attention mass per (query block, KV block): [B, H, N/Bq, N/Bk] float32.

    With ``rep_row`` the representative-row variant: the mass of the single row
    qb * q_block + rep_row of each query block (rows sum to 1).  ``return_projections`` also
    returns the two operands of the logit product: Q~ = round(pred_scale * log2(e) * q @ wq) (the
    scale applied before the one rounding) and K_lr = round(k @ wk); logit = ln(2) * <Q~_i, K_lr_j>."""
    lib = load_library()
    b, h, n, d, r = _predict_inputs(q, k, wq, wk)
    nqb, nkb = _blocks(n, q_block, kv_block)
    if out is not None:
        _expect(out, "out", (b, h, nqb, nkb), torch.float32)
    dev = _dev(q, k, wq, wk, out)
    prob = make_problem(q, q_block=q_block, kv_block=kv_block, topk=1, rank=r, pred_scale=pred_scale)
    ws = _workspace(int(lib.dsv_predict_workspace_size(ctypes.byref(prob))), dev, workspace)
    scores = out if out is not None else torch.empty((b, h, nqb, nkb), dtype=torch.float32, device=dev)
    nbytes = ws.numel() * ws.element_size()
    if rep_row is None:
        _check(lib.dsv_predict(ctypes.byref(prob), _p(q), _p(k), _p(wq), _p(wk), _p(ws), nbytes, _p(scores),
                               _stream(dev)), "dsv_predict")
    else:
        _check(lib.dsv_predict_representative(ctypes.byref(prob), _p(q), _p(k), _p(wq), _p(wk), int(rep_row), _p(ws),
                                              nbytes, _p(scores), _stream(dev)), "dsv_predict_representative")
    if return_projections:
        return (scores, *_projections(ws, q, b, h, n, r))
    return scores


def predict_select_representative(q, k, wq, wk, topk: int, rep_row: int, *, q_block: int, kv_block: int = 64,
                                  pred_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                                  return_projections: bool = False, out: Optional[torch.Tensor] = None):
    """The fused representative-row predictor and top-k: for every query block, the ``topk`` KV
    blocks with the largest predicted mass of its row qb * q_block + rep_row, ascending ->
    block_idx [B, H, N/Bq, k] int32 (no score matrix is formed).  ``return_projections`` also
    returns Q~ and K_lr as :func:`predict` does."""
    lib = load_library()
    b, h, n, d, r = _predict_inputs(q, k, wq, wk)
    nqb, nkb = _blocks(n, q_block, kv_block)
    if out is not None:
        _expect(out, "out", (b, h, nqb, topk), torch.int32)
    dev = _dev(q, k, wq, wk, out)
    prob = make_problem(q, q_block=q_block, kv_block=kv_block, topk=topk, rank=r, pred_scale=pred_scale)
    ws = _workspace(int(lib.dsv_predict_workspace_size(ctypes.byref(prob))), dev, workspace)
    idx = out if out is not None else torch.empty((b, h, nqb, topk), dtype=torch.int32, device=dev)
    _check(lib.dsv_predict_select_representative(ctypes.byref(prob), _p(q), _p(k), _p(wq), _p(wk), int(rep_row),
                                                 _p(ws), ws.numel() * ws.element_size(), _p(idx), _stream(dev)),
           "dsv_predict_select_representative")
    if return_projections:
        return (idx, *_projections(ws, q, b, h, n, r))
    return idx


def _scores_shape(scores: torch.Tensor, q_block: int, kv_block: int):
    if scores.dtype != torch.float32 or scores.dim() != 4:
        raise TypeError("scores must be float32 [B, H, N/Bq, N/Bk]")
    _contig(scores)
    b, h, nqb, nkb = scores.shape
    n = nkb * kv_block
    if nqb * q_block != n:
        raise ValueError("scores shape does not match the block sizes")
    return b, h, nqb, nkb, n


def select_topk(scores: torch.Tensor, topk: int, *, q_block: int, kv_block: int = 64,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The top-k KV blocks of every query block, ascending, ties to the smaller index."""
    lib = load_library()
    b, h, nqb, nkb, n = _scores_shape(scores, q_block, kv_block)
    if out is not None:
        _expect(out, "out", (b, h, nqb, topk), torch.int32)
    dev = _dev(scores, out)
    prob = Problem(b, h, n, 64, q_block, kv_block, topk, 1, DSV_F32, 0.0, 0.0)
    idx = out if out is not None else torch.empty((b, h, nqb, topk), dtype=torch.int32, device=dev)
    _check(lib.dsv_select_topk(ctypes.byref(prob), _p(scores), _p(idx), _stream(dev)), "dsv_select_topk")
    return idx


def select_mass(scores: torch.Tensor, tau: float, kmax: int, *, q_block: int, kv_block: int = 64,
                out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The fewest KV blocks (by descending score) carrying a fraction tau of each query block's
    score, at most kmax -> (block_idx ascending then -1 padding, block_counts)."""
    lib = load_library()
    b, h, nqb, nkb, n = _scores_shape(scores, q_block, kv_block)
    if out is not None:
        idx, cnt = out
        _expect(idx, "out[0] (block_idx)", (b, h, nqb, kmax), torch.int32)
        _expect(cnt, "out[1] (block_counts)", (b, h, nqb), torch.int32)
        dev = _dev(scores, idx, cnt)
    else:
        dev = _dev(scores)
        idx = torch.empty((b, h, nqb, kmax), dtype=torch.int32, device=dev)
        cnt = torch.empty((b, h, nqb), dtype=torch.int32, device=dev)
    prob = Problem(b, h, n, 64, q_block, kv_block, kmax, 1, DSV_F32, 0.0, 0.0)
    _check(lib.dsv_select_mass(ctypes.byref(prob), _p(scores), ctypes.c_float(tau), _p(idx), _p(cnt), _stream(dev)),
           "dsv_select_mass")
    return idx, cnt


def _attn_inputs(q, k, v, block_idx, q_block, kv_block):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    b, h, n, d = q.shape
    _dtype_code(q)
    _contig(q)
    _expect(k, "k", q.shape, q.dtype)
    _expect(v, "v", q.shape, q.dtype)
    nqb, _ = _blocks(n, q_block, kv_block)
    if block_idx.dim() != 4:
        raise ValueError("block_idx must be [B, H, N/Bq, k]")
    _expect(block_idx, "block_idx", (b, h, nqb, block_idx.shape[-1]), torch.int32)
    return b, h, n, d


def sparse_attn_fwd(q, k, v, block_idx, *, q_block: int, kv_block: int = 64, sm_scale: Optional[float] = None,
                    block_counts: Optional[torch.Tensor] = None, residual: bool = False,
                    workspace: Optional[torch.Tensor] = None, out=None):
    """Softmax attention over the selected KV blocks only -> (o [B,H,N,d], lse [B,H,N] float32).

    With ``residual=True`` (bf16 only) also returns o_lo, the bf16 rounding residual of O; handing it
    to :func:`sparse_attn_bwd` makes the backward's D = rowsum(dO * O) accurate.  This training
    forward needs a workspace (an fp16 copy of V); the inference forward needs none.
    ``out`` may supply (o, lse) or (o, lse, o_lo).  ``block_counts`` ([B, H, N/Bq] int32, e.g. from
    :func:`select_mass`) limits each query block to the first entries of its list.
    """
    lib = load_library()
    b, h, n, d = _attn_inputs(q, k, v, block_idx, q_block, kv_block)
    if residual and q.dtype != torch.bfloat16:
        raise ValueError("the O residual exists for bf16 problems only")
    _check_counts(block_counts, block_idx)
    o_lo = None
    if out is not None:
        if len(out) < (3 if residual else 2):
            raise ValueError("out must hold (o, lse) or, with residual=True, (o, lse, o_lo)")
        o, lse = out[0], out[1]
        _expect(o, "out[0] (o)", q.shape, q.dtype)
        _expect(lse, "out[1] (lse)", (b, h, n), torch.float32)
        if residual:
            o_lo = out[2]
            _expect(o_lo, "out[2] (o_lo)", q.shape, torch.bfloat16)
        dev = _dev(q, k, v, block_idx, block_counts, o, lse, o_lo)
    else:
        dev = _dev(q, k, v, block_idx, block_counts)
        o = torch.empty_like(q)
        lse = torch.empty((b, h, n), dtype=torch.float32, device=dev)
        if residual:
            o_lo = torch.empty_like(q)
    prob = make_problem(q, q_block=q_block, kv_block=kv_block, topk=block_idx.shape[-1], sm_scale=sm_scale)
    ws = _workspace(int(lib.dsv_sparse_attn_fwd_workspace_size(ctypes.byref(prob))) if residual else 0, dev,
                    workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dsv_sparse_attn_fwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(block_idx), _p(block_counts), _p(o),
                                   _p(lse), _p(o_lo), _p(ws), nbytes, _stream(dev)), "dsv_sparse_attn_fwd")
    return (o, lse, o_lo) if residual else (o, lse)


def sparse_attn_bwd(q, k, v, o, dout, lse, block_idx, *, q_block: int, kv_block: int = 64,
                    sm_scale: Optional[float] = None, o_lo: Optional[torch.Tensor] = None,
                    block_counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Gradients (dq, dk, dv) of the sparse attention; ``o_lo`` is the forward's residual (or None)."""
    lib = load_library()
    b, h, n, d = _attn_inputs(q, k, v, block_idx, q_block, kv_block)
    _expect(o, "o", q.shape, q.dtype)
    _expect(dout, "dout", q.shape, q.dtype)
    _expect(lse, "lse", (b, h, n), torch.float32)
    if o_lo is not None:
        _expect(o_lo, "o_lo", q.shape, torch.bfloat16)
    _check_counts(block_counts, block_idx)
    if out is not None:
        dq, dk, dv = out
        for nm, t in (("out[0] (dq)", dq), ("out[1] (dk)", dk), ("out[2] (dv)", dv)):
            _expect(t, nm, q.shape, q.dtype)
    dev = _dev(q, k, v, o, dout, lse, block_idx, o_lo, block_counts, *(out or ()))
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    prob = make_problem(q, q_block=q_block, kv_block=kv_block, topk=block_idx.shape[-1], sm_scale=sm_scale)
    ws = _workspace(int(lib.dsv_sparse_attn_bwd_workspace_size(ctypes.byref(prob))), dev, workspace)
    _check(lib.dsv_sparse_attn_bwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(o), _p(o_lo), _p(dout), _p(lse),
                                   _p(block_idx), _p(block_counts), _p(dq), _p(dk), _p(dv), _p(ws),
                                   ws.numel() * ws.element_size(), _stream(dev)), "dsv_sparse_attn_bwd")
    return dq, dk, dv


def head_density(block_counts: Optional[torch.Tensor], *, topk: int, seq_len: int, q_block: int, kv_block: int = 64,
                 dense_above: float = 0.5, batch: Optional[int] = None, heads: Optional[int] = None):
    """Per-head selected density and dense flag (the per-block activation of sparse attention):
    density = selected KV blocks / (N/Bq * N/Bk); dense = 1 where the selected count exceeds
    floor(dense_above * N/Bq * N/Bk).  block_counts [B, H, N/Bq] int32, or None with batch, heads
    given (every list full).  Returns (density float32 [B, H], dense int32 [B, H])."""
    lib = load_library()
    if block_counts is not None:
        if block_counts.dim() != 3:
            raise ValueError("block_counts must be int32 [B, H, N/Bq]")
        batch, heads = block_counts.shape[0], block_counts.shape[1]
        _expect(block_counts, "block_counts", (batch, heads, seq_len // q_block), torch.int32)
        dev = _dev(block_counts)
    else:
        if batch is None or heads is None:
            raise ValueError("without block_counts, pass batch and heads")
        dev = torch.device("cuda", torch.cuda.current_device())
    prob = Problem(batch, heads, seq_len, 64, q_block, kv_block, topk, 1, DSV_BF16, 0.0, 0.0)
    density = torch.empty((batch, heads), dtype=torch.float32, device=dev)
    dense = torch.empty((batch, heads), dtype=torch.int32, device=dev)
    _check(lib.dsv_head_density(ctypes.byref(prob), _p(block_counts), ctypes.c_float(dense_above), _p(density),
                                _p(dense), _stream(dev)), "dsv_head_density")
    return density, dense


def block_recall(lse_selected: torch.Tensor, lse_all: torch.Tensor, *, q_block: int,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mean over each query block's rows of exp(lse_selected - lse_all): the true attention mass
    the selection captures (lse_all from the forward with every block selected)."""
    lib = load_library()
    if lse_selected.dim() != 3:
        raise ValueError("lse tensors must be float32 [B, H, N]")
    b, h, n = lse_selected.shape
    _expect(lse_selected, "lse_selected", (b, h, n), torch.float32)
    _expect(lse_all, "lse_all", (b, h, n), torch.float32)
    if n % q_block:
        raise ValueError("N must be a multiple of q_block")
    if out is not None:
        _expect(out, "out", (b, h, n // q_block), torch.float32)
    dev = _dev(lse_selected, lse_all, out)
    prob = Problem(b, h, n, 64, q_block, q_block, 1, 1, DSV_F32, 0.0, 0.0)
    rec = out if out is not None else torch.empty((b, h, n // q_block), dtype=torch.float32, device=dev)
    _check(lib.dsv_block_recall(ctypes.byref(prob), _p(lse_selected), _p(lse_all), _p(rec), _stream(dev)),
           "dsv_block_recall")
    return rec


def pack_kv(k, v, block_idx, qb_begin: int, qb_end: int, *, q_block: int, kv_block: int = 64,
            block_counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Pack the KV blocks selected by query blocks [qb_begin, qb_end) for sequence sharding ->
    (k_packed, v_packed [B,H,N,d], packed_blocks [B,H,N/Bk], packed_counts [B,H],
    packed_idx [B,H,qb_end-qb_begin,k])."""
    lib = load_library()
    b, h, n, d = _attn_inputs(k, k, v, block_idx, q_block, kv_block)
    _check_counts(block_counts, block_idx)
    dev = _dev(k, v, block_idx, block_counts)
    prob = make_problem(k, q_block=q_block, kv_block=kv_block, topk=block_idx.shape[-1])
    ws = _workspace(int(lib.dsv_pack_kv_workspace_size(ctypes.byref(prob))), dev, workspace)
    kp, vp = torch.empty_like(k), torch.empty_like(v)
    blocks = torch.empty((b, h, n // kv_block), dtype=torch.int32, device=dev)
    counts = torch.empty((b, h), dtype=torch.int32, device=dev)
    pidx = torch.empty((b, h, max(qb_end - qb_begin, 0), block_idx.shape[-1]), dtype=torch.int32, device=dev)
    _check(lib.dsv_pack_kv(ctypes.byref(prob), _p(k), _p(v), _p(block_idx), _p(block_counts), int(qb_begin),
                           int(qb_end), _p(kp), _p(vp), _p(blocks), _p(counts), _p(pidx) if pidx.numel() else None,
                           _p(ws), ws.numel() * ws.element_size(), _stream(dev)), "dsv_pack_kv")
    return kp, vp, blocks, counts, pidx


def pack_kv_noalloc(k, v, block_idx, qb_begin: int, qb_end: int, *, out, q_block: int, kv_block: int = 64,
                    block_counts: Optional[torch.Tensor] = None):
    """:func:`pack_kv` with no allocation at all: ``out`` = (k_packed, v_packed, packed_blocks,
    packed_counts, packed_idx), shaped as pack_kv returns them, is filled in place (packed_idx may
    be None when qb_end == qb_begin).  The scratch is the library's own device array (B*H*N/Bk <=
    262144); calls that overlap in time on one GPU race."""
    lib = load_library()
    kp, vp, blocks, counts, pidx = out
    dev = _dev(k, v, block_idx, kp, vp, blocks, counts)
    _contig(k, v, block_idx, kp, vp, blocks, counts, pidx)
    b, h, n, d = k.shape
    nsh = max(qb_end - qb_begin, 0)
    want = {"k_packed": (kp, k.shape, k.dtype), "v_packed": (vp, k.shape, k.dtype),
            "packed_blocks": (blocks, (b, h, n // kv_block), torch.int32), "packed_counts": (counts, (b, h), torch.int32)}
    if nsh:
        want["packed_idx"] = (pidx, (b, h, nsh, block_idx.shape[-1]), torch.int32)
    for name, (t, shape, dt) in want.items():
        if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dt or t.device != dev:
            raise ValueError(f"{name} must be {dt} {tuple(shape)} on {dev}")
    prob = make_problem(k, q_block=q_block, kv_block=kv_block, topk=block_idx.shape[-1])
    _check_counts(block_counts, block_idx)
    _check(lib.dsv_pack_kv_noalloc(ctypes.byref(prob), _p(k), _p(v), _p(block_idx), _p(block_counts), int(qb_begin),
                                   int(qb_end), _p(kp), _p(vp), _p(blocks), _p(counts), _p(pidx) if nsh else None,
                                   _stream(dev)), "dsv_pack_kv_noalloc")
    return kp, vp, blocks, counts, pidx


def workspace_sizes(q: torch.Tensor, *, q_block: int, kv_block: int, topk: int, rank: int):
    """(predict, forward, backward) workspace bytes for a problem shaped like q."""
    lib = load_library()
    prob = make_problem(q, q_block=q_block, kv_block=kv_block, topk=topk, rank=rank)
    return (int(lib.dsv_predict_workspace_size(ctypes.byref(prob))),
            int(lib.dsv_sparse_attn_fwd_workspace_size(ctypes.byref(prob))),
            int(lib.dsv_sparse_attn_bwd_workspace_size(ctypes.byref(prob))))


PEAK_KINDS = {"mfma_bf16": 0, "mfma_f16": 1, "exp_f32": 2, "hbm_copy": 3, "hbm_read": 4}


def peak_probe(kind: str, repeats: int = 5, device: Optional[torch.device] = None) -> float:
    """Sustained rate of one operation on this device (blocks): ``mfma_bf16`` / ``mfma_f16`` in
    flop/s (MFMA 32x32x16), ``exp_f32`` in exponentials/s, ``hbm_copy`` in bytes/s read + written,
    ``hbm_read`` in bytes/s read."""
    lib = load_library()
    code = PEAK_KINDS[kind]
    dev = device or torch.device("cuda", torch.cuda.current_device())
    nbytes = int(lib.dsv_peak_probe_workspace_size(code))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rate = ctypes.c_double(0.0)
    _check(lib.dsv_peak_probe(code, int(repeats), _p(ws), nbytes, ctypes.byref(rate), _stream(dev)), "dsv_peak_probe")
    return rate.value


def timing_begin() -> None:
    """Start bracketing every library launch from this thread with HIP events."""
    _check(load_library().dsv_timing_begin(), "dsv_timing_begin")


def timing_end() -> dict:
    """Stop timing; {kernel name: (launches, total_ms, min_ms, max_ms)} (synchronises on the events)."""
    lib = load_library()
    buf = (KernelStat * 64)()
    n = lib.dsv_timing_end(buf, 64)
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms, buf[i].min_ms, buf[i].max_ms)
            for i in range(min(n, 64))}


class DSVAttention(torch.autograd.Function):
    """predict -> select -> sparse forward; the backward is the sparse backward.

    No gradient flows to the predictor weights or the selection.
    """

    @staticmethod
    def forward(ctx, q, k, v, wq, wk, q_block: int, kv_block: int, topk: int, sm_scale=None, pred_scale=None):
        scores = predict(q, k, wq, wk, q_block=q_block, kv_block=kv_block, pred_scale=pred_scale)
        idx = select_topk(scores, topk, q_block=q_block, kv_block=kv_block)
        res = q.dtype == torch.bfloat16
        out = sparse_attn_fwd(q, k, v, idx, q_block=q_block, kv_block=kv_block, sm_scale=sm_scale, residual=res)
        o, lse = out[0], out[1]
        ctx.save_for_backward(q, k, v, o, lse, idx, *out[2:])
        ctx.cfg = (q_block, kv_block, sm_scale)
        ctx.mark_non_differentiable(idx)
        return o, idx

    @staticmethod
    def backward(ctx, do, _didx):
        q, k, v, o, lse, idx, *o_lo = ctx.saved_tensors
        qb, kb, sm = ctx.cfg
        dq, dk, dv = sparse_attn_bwd(q, k, v, o, do.contiguous(), lse, idx, q_block=qb, kv_block=kb, sm_scale=sm,
                                     o_lo=o_lo[0] if o_lo else None)
        return dq, dk, dv, None, None, None, None, None, None, None
