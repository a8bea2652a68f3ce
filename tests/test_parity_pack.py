"""GPU parity of the KV packing for sequence sharding: the packed union, counts and rewritten
lists equal the oracle's exactly (integer work), the packed rows are the original rows byte for
byte, and the forward over the packed buffer equals the forward over the original K/V bit for bit
(the same kernel reads the same blocks in the same order)."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from oracle import dsv_oracle as O
from tests.gpu_helpers import log, to_dev
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsv.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,ragged,qb0,qb1", [("C2", False, 32, 48), ("C2", True, 0, 128), ("C3", False, 100, 101),
                                                 ("C2", True, 7, 7), ("C1", False, 4, 12)])
def test_pack_matches_the_oracle_and_the_forward_is_unchanged(name, ragged, qb0, qb1):
    cfg = get_config(name)
    cfg = cfg.with_(heads=min(cfg.heads, 3))
    inp = make_inputs(cfg, with_grad=False)
    t = {k: to_dev(v) for k, v in inp.items()}
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block)
    scores = dsv.predict(t["q"], t["k"], t["wq"], t["wk"], **kw)
    if ragged:
        idx, cnt = dsv.select_mass(scores, 0.3, min(2 * cfg.topk, cfg.nkb), **kw)
    else:
        idx, cnt = dsv.select_topk(scores, cfg.topk, **kw), None
    kp, vp, blocks, counts, pidx = dsv.pack_kv(t["k"], t["v"], idx, qb0, qb1, block_counts=cnt, **kw)
    torch.cuda.synchronize()
    cnt_np = None if cnt is None else cnt.cpu().numpy()
    rb, rc, rr = O.pack_selected(idx.cpu().numpy(), cnt_np, qb0, qb1, cfg.nkb)
    assert np.array_equal(blocks.cpu().numpy(), rb) and np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(pidx.cpu().numpy(), rr)
    log(f"[parity] pack {name} query blocks [{qb0}, {qb1}): union sizes {rc.ravel().tolist()} of {cfg.nkb}")
    for h in range(cfg.heads):
        for u in range(int(rc[0, h])):
            kb = int(rb[0, h, u])
            src, dst = slice(kb * 64, kb * 64 + 64), slice(u * 64, u * 64 + 64)
            assert torch.equal(kp[0, h, dst], t["k"][0, h, src]) and torch.equal(vp[0, h, dst], t["v"][0, h, src])
    if qb1 == qb0:
        return
    # the receiver's forward over the packed buffer: its Q rows, the rewritten lists
    rows = slice(qb0 * cfg.q_block, qb1 * cfg.q_block)
    q_sh = t["q"][:, :, rows].contiguous()
    zero_pad = torch.zeros_like(t["q"])
    zero_pad[:, :, : qb1 * cfg.q_block - qb0 * cfg.q_block] = q_sh
    nsh = qb1 - qb0
    full_idx = torch.zeros_like(idx)
    full_idx[:, :, :nsh] = pidx.clamp(min=0)
    full_cnt = torch.zeros(idx.shape[:-1], dtype=torch.int32, device=idx.device)
    full_cnt[:, :, :nsh] = cnt[:, :, qb0:qb1] if cnt is not None else idx.shape[-1]
    o_p, l_p = dsv.sparse_attn_fwd(zero_pad, kp, vp, full_idx, block_counts=full_cnt, **kw)
    o_r, l_r = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, block_counts=cnt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_p[:, :, :nsh * cfg.q_block], o_r[:, :, rows])
    assert torch.equal(l_p[:, :, :nsh * cfg.q_block], l_r[:, :, rows])
