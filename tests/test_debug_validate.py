"""The opt-in device check of block lists (DSV_DEBUG_VALIDATE=1): the attention calls are defined
only for lists whose used entries are distinct indices in [0, N/Bk).  With the check on, a list
with a repeated or out-of-range entry is refused with DSV_ERR_INVALID_ARGUMENT before any
attention kernel runs; valid lists (ragged ones with -1 padding past their counts included) give
the same outputs as without the check."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from tests.gpu_helpers import log, seeded_idx, to_dev
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture()
def checked(monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsv.load_library()
    monkeypatch.setenv("DSV_DEBUG_VALIDATE", "1")
    yield
    torch.cuda.synchronize()


def test_debug_check_refuses_bad_lists_and_passes_good_ones(checked, monkeypatch):
    cfg = get_config("C2").with_(heads=2, latent=(4, 16, 16), topk=4)  # N = 1024, 16 KV blocks
    inp = make_inputs(cfg)
    t = {k: to_dev(v) for k, v in inp.items()}
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block)
    good = seeded_idx(3, (1, 2), cfg.nqb, cfg.nkb, cfg.topk)
    o, lse = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], to_dev(good), **kw)
    g = dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, to_dev(good), **kw)
    # ragged: -1 padding past each count is never read, so it passes
    cnt = np.full((1, 2, cfg.nqb), 3, np.int32)
    ragged = good.copy()
    ragged[..., 3] = -1
    dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], to_dev(ragged), block_counts=to_dev(cnt), **kw)
    for name, bad in (("repeat", 0), ("out of range", 1), ("negative within the count", 2)):
        b = good.copy()
        if bad == 0:
            b[0, 1, 5, 2] = b[0, 1, 5, 0]
        elif bad == 1:
            b[0, 0, 7, 3] = cfg.nkb
        else:
            b[0, 0, 2, 1] = -1
        for call in ("fwd", "bwd"):
            with pytest.raises(dsv.DSVError) as e:
                if call == "fwd":
                    dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], to_dev(b), **kw)
                else:
                    dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, to_dev(b), **kw)
            assert e.value.status == 1 and "DSV_DEBUG_VALIDATE" in str(e.value), str(e.value)
        log(f"[debug-check] {name}: refused by the forward and the backward")
    # the checked results equal the unchecked ones
    monkeypatch.delenv("DSV_DEBUG_VALIDATE")
    o2, lse2 = dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], to_dev(good), **kw)
    g2 = dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o2, t["do"], lse2, to_dev(good), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and all(torch.equal(a, b) for a, b in zip(g, g2))
