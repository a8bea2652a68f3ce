"""The allocation-free entry point dsv_pack_kv_noalloc against dsv_pack_kv: the same outputs,
bit for bit, on two calls in a row (the second smaller, with other lists), so that the
library's shared device scratch carries nothing from one call into the next."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv
from tests.gpu_helpers import log, seeded_idx, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, b, h, n, d, k, qb0, qb1, ragged):
    rng = np.random.default_rng(seed)
    kk = torch.from_numpy(rng.standard_normal((b, h, n, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    vv = torch.from_numpy(rng.standard_normal((b, h, n, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    nqb, nkb = n // 128, n // 64
    idx = seeded_idx(seed, (b, h), nqb, nkb, k)
    cnt = None
    if ragged:
        c = rng.integers(0, k + 1, size=(b, h, nqb)).astype(np.int32)
        for bi in range(b):
            for hi in range(h):
                for q in range(nqb):
                    idx[bi, hi, q, c[bi, hi, q]:] = -1
        cnt = to_dev(c)
    return kk, vv, to_dev(idx), cnt


def _compare(kk, vv, idx, cnt, qb0, qb1):
    ref = dsv.pack_kv(kk, vv, idx, qb0, qb1, q_block=128, block_counts=cnt)
    b, h, n, d = kk.shape
    # outputs pre-filled with garbage: everything the call defines must be overwritten
    out = (torch.full_like(kk, 7.0), torch.full_like(vv, -3.0),
           torch.full((b, h, n // 64), 12345, dtype=torch.int32, device="cuda"),
           torch.full((b, h), -9, dtype=torch.int32, device="cuda"),
           torch.full((b, h, qb1 - qb0, idx.shape[-1]), 777, dtype=torch.int32, device="cuda"))
    got = dsv.pack_kv_noalloc(kk, vv, idx, qb0, qb1, q_block=128, block_counts=cnt, out=out)
    torch.cuda.synchronize()
    assert torch.equal(got[2], ref[2]) and torch.equal(got[3], ref[3]) and torch.equal(got[4], ref[4])
    counts = ref[3].cpu().numpy()
    for bi in range(b):
        for hi in range(h):
            rows = int(counts[bi, hi]) * 64  # rows past the union are not written by either call
            assert torch.equal(got[0][bi, hi, :rows], ref[0][bi, hi, :rows])
            assert torch.equal(got[1][bi, hi, :rows], ref[1][bi, hi, :rows])
    return counts


def test_noalloc_pack_matches_the_workspace_call_on_calls_in_a_row():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsv.load_library()
    # exactly at the scratch limit: B*H*N/Bk = 64 * 4096 = 262144 entries (K, V drawn on the device)
    log("[noalloc] call at the limit: B=1 H=64 N=262144 d=64 k=4, query blocks [0, 16)")
    g = torch.Generator(device="cuda").manual_seed(1)
    kk = torch.randn((1, 64, 262144, 64), generator=g, device="cuda").to(torch.bfloat16)
    vv = torch.randn((1, 64, 262144, 64), generator=g, device="cuda").to(torch.bfloat16)
    c0 = _compare(kk, vv, to_dev(seeded_idx(2, (1, 64), 2048, 4096, 4)), None, 0, 16)
    del kk, vv
    log("[noalloc] second call, smaller: B=2 H=20 N=16384 d=128 k=26, query blocks [16, 112)")
    c1 = _compare(*_case(3, 2, 20, 16384, 128, 26, 16, 112, ragged=False), 16, 112)
    log("[noalloc] third call, smaller: B=1 H=3 N=4096 d=64 k=5 ragged, query blocks [0, 9)")
    c2 = _compare(*_case(4, 1, 3, 4096, 64, 5, 0, 9, ragged=True), 0, 9)
    assert c1.max() > c2.max()  # the later union is smaller: stale flags from before would show
    log(f"[noalloc] unions {c0.min()}..{c0.max()}, {c1.min()}..{c1.max()}, {c2.min()}..{c2.max()} blocks: "
        "equal to dsv_pack_kv")
