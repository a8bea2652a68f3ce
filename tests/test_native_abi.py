"""The C ABI driven from C++ (tests/native/abi_roundtrip.cpp): the whole hot path -- predict,
top-k, the training forward and the backward -- with plain hipMalloc'd buffers and the null
stream, no Python or torch in the caller.  Its outputs must equal the Python binding's bit for
bit: the same kernels, which are deterministic."""
import os
import subprocess

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from tests.gpu_helpers import log, to_dev
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_roundtrip")


def test_native_caller_matches_the_binding(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "tests/native/abi_roundtrip is not built (the library build makes it)"
    dsv.load_library()
    cfg = get_config("C3").with_(heads=3)  # d = 128, Bq = 64, r = 32
    inp = make_inputs(cfg, with_grad=True)
    b, h, n, d, r = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.rank
    raw = np.concatenate([inp[nm].reshape(-1) for nm in ("q", "k", "v", "do", "wq", "wk")]).astype(np.uint16)
    (tmp_path / "in.bin").write_bytes(raw.tobytes())
    args = [BIN, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")] + [str(x) for x in
                                                                          (b, h, n, d, r, cfg.q_block, cfg.topk)]
    res = subprocess.run(args, capture_output=True, text=True, timeout=120)
    log(f"[parity] native caller: {res.stdout.strip()} {res.stderr.strip()}")
    assert res.returncode == 0, res.stderr

    out = np.frombuffer((tmp_path / "out.bin").read_bytes(), dtype=np.uint8)
    act = b * h * n * d
    layout = [("scores", np.float32, b * h * cfg.nqb * cfg.nkb), ("idx", np.int32, b * h * cfg.nqb * cfg.topk),
              ("o", np.uint16, act), ("lse", np.float32, b * h * n), ("dq", np.uint16, act), ("dk", np.uint16, act),
              ("dv", np.uint16, act)]
    native, off = {}, 0
    for nm, dt, cnt in layout:
        nbytes = cnt * np.dtype(dt).itemsize
        native[nm] = out[off:off + nbytes].view(dt)
        off += nbytes
    assert off == out.size

    t = {k: to_dev(v) for k, v in inp.items()}
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block)
    scores = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], **kw)
    idx = dsv.select_topk(scores, cfg.topk, **kw)
    o, lse, o_lo = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, residual=True, **kw)
    dq, dk, dv = dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, idx, o_lo=o_lo, **kw)
    torch.cuda.synchronize()

    def bits(x):
        x = x.detach().cpu().contiguous()
        return (x.view(torch.int16) if x.dtype == torch.bfloat16 else x).numpy().reshape(-1).view(
            {torch.bfloat16: np.uint16, torch.float32: np.float32, torch.int32: np.int32}[x.dtype])

    for nm, got in (("scores", scores), ("idx", idx), ("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.array_equal(native[nm].view(np.uint8), bits(got).view(np.uint8)), nm
