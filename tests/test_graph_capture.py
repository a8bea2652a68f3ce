"""The whole step -- predict, select, training forward, backward -- captured once in a HIP graph
(torch.cuda.graph) and replayed.  The library only enqueues kernels on the caller's stream,
allocates nothing and clears its scratch with fill kernels rather than memset nodes, so a captured
step must reproduce the eager one bit for bit on every replay, also with other eager work and
synchronisations between the replays and new input values copied into the captured buffers."""
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from tests.gpu_helpers import log, to_dev
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def test_captured_step_replays_equal_the_eager_step():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsv.load_library()
    cfg = get_config("C2").with_(heads=4)  # N = 8192, d = 64, Bq = 64, k = 13
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block)
    inputs = [{k: to_dev(v) for k, v in make_inputs(cfg.with_(seed=cfg.seed + i)).items()} for i in range(3)]
    t = {k: v.clone() for k, v in inputs[0].items()}  # the captured buffers
    B, H, N, D = t["q"].shape
    ws_p, ws_f, ws_b = dsv.workspace_sizes(t["q"], topk=cfg.topk, rank=cfg.rank, **kw)
    wsp = torch.empty(ws_p, dtype=torch.uint8, device="cuda")
    wsf = torch.empty(ws_f, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    scores = torch.empty((B, H, cfg.nqb, cfg.nkb), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, H, cfg.nqb, cfg.topk), dtype=torch.int32, device="cuda")
    o, o_lo = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(t["q"]) for _ in range(3))

    def step():
        dsv.predict(t["q"], t["k"], t["wq"], t["wk"], workspace=wsp, out=scores, **kw)
        dsv.select_topk(scores, cfg.topk, out=idx, **kw)
        dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, workspace=wsf, residual=True, out=(o, lse, o_lo), **kw)
        dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, idx, o_lo=o_lo, workspace=wsb, out=grads, **kw)

    def snapshot():
        return [x.clone() for x in (scores, idx, o, lse, o_lo, *grads)]

    # eager reference for each input set
    want = []
    for inp in inputs:
        for k in t:
            t[k].copy_(inp[k])
        step()
        torch.cuda.synchronize()
        want.append(snapshot())
    # capture (after a warm-up on a side stream, as torch requires)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    names = ("scores", "idx", "o", "lse", "o_lo", "dq", "dk", "dv")
    for rep in range(6):
        which = rep % 3
        for k in t:
            t[k].copy_(inputs[which][k])
        for x in (scores, idx, o, lse, o_lo, *grads):  # stale values must not survive a replay
            x.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for nm, a, b in zip(names, got, want[which]):
            assert torch.equal(a, b), f"replay {rep} (inputs {which}): {nm} differs from the eager step"
        # eager work of the program's own between replays
        step()
        torch.cuda.synchronize()
    log("[graph] 6 replays of the captured step over 3 input sets equal the eager step bit for bit")
