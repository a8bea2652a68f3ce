"""The Python binding refuses tensors whose shape or dtype would make a kernel read or write
outside an allocation -- inputs and out= buffers alike -- with a ValueError raised before any
device work.  CPU tensors with valid shapes get past these checks and are then refused because
no CPU path exists, which shows that the checks come first."""
import os

import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv

B, H, N, D, R, BQ, K = 1, 2, 1024, 64, 16, 64, 3
NQB, NKB = N // BQ, N // 64


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(dsv.LIB_PATH):
        pytest.skip("libdsv.so not built")
    return dsv.load_library()


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def good():
    return dict(q=bf(B, H, N, D), k=bf(B, H, N, D), v=bf(B, H, N, D), o=bf(B, H, N, D), do=bf(B, H, N, D),
                lse=f32(B, H, N), idx=i32(B, H, NQB, K), wq=bf(H, D, R), wk=bf(H, D, R))


def no_gpu(fn):
    with pytest.raises(RuntimeError, match="GPU tensors"):
        fn()


def test_valid_cpu_tensors_pass_validation_and_then_find_no_cpu_path():
    t = good()
    no_gpu(lambda: dsv.predict(t["q"], t["k"], t["wq"], t["wk"], q_block=BQ))
    no_gpu(lambda: dsv.predict_select_representative(t["q"], t["k"], t["wq"], t["wk"], K, 0, q_block=BQ))
    no_gpu(lambda: dsv.select_topk(f32(B, H, NQB, NKB), K, q_block=BQ))
    no_gpu(lambda: dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], t["idx"], q_block=BQ))
    no_gpu(lambda: dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["idx"], q_block=BQ))


@pytest.mark.parametrize("name,bad", [("k", bf(B, H, N, 32)), ("k", torch.zeros(B, H, N, D)),
                                      ("v", bf(B, H, N // 2, D)), ("idx", torch.zeros(B, H, NQB, K, dtype=torch.int64)),
                                      ("idx", i32(B, H, NQB + 1, K))])
def test_forward_rejects_mismatched_inputs(name, bad):
    t = good()
    t[name] = bad
    with pytest.raises(ValueError):
        dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], t["idx"], q_block=BQ)


@pytest.mark.parametrize("which,bad", [(0, bf(B, H, N, 32)), (1, f32(B, H, N - 64)), (1, bf(B, H, N)),
                                       (2, f32(B, H, N, D))])
def test_forward_rejects_mismatched_out_buffers(which, bad):
    t = good()
    out = [bf(B, H, N, D), f32(B, H, N), bf(B, H, N, D)]
    out[which] = bad
    with pytest.raises(ValueError):
        dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], t["idx"], q_block=BQ, residual=True, out=tuple(out))
    with pytest.raises(ValueError):  # a residual forward needs three out buffers
        dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], t["idx"], q_block=BQ, residual=True, out=tuple(out[:2]))


@pytest.mark.parametrize("name,bad", [("o", bf(B, H, N, 32)), ("do", bf(B, H, N - 64, D)), ("do", f32(B, H, N, D)),
                                      ("lse", f32(B, H, N - 1)), ("lse", bf(B, H, N)), ("k", f32(B, H, N, D))])
def test_backward_rejects_mismatched_inputs(name, bad):
    t = good()
    t[name] = bad
    with pytest.raises(ValueError):
        dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["idx"], q_block=BQ)


def test_backward_rejects_bad_residual_counts_and_out_buffers():
    t = good()
    args = (t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["idx"])
    with pytest.raises(ValueError):
        dsv.sparse_attn_bwd(*args, q_block=BQ, o_lo=f32(B, H, N, D))
    with pytest.raises(ValueError):
        dsv.sparse_attn_bwd(*args, q_block=BQ, block_counts=i32(B, H, NQB - 1))
    with pytest.raises(ValueError):
        dsv.sparse_attn_bwd(*args, q_block=BQ, out=(bf(B, H, N, D), bf(B, H, N, D), bf(B, H, N // 2, D)))
    with pytest.raises(ValueError):
        dsv.sparse_attn_bwd(*args, q_block=BQ, out=(f32(B, H, N, D), bf(B, H, N, D), bf(B, H, N, D)))


def test_predictor_and_selection_reject_mismatched_tensors():
    t = good()
    with pytest.raises(ValueError):
        dsv.predict(t["q"], bf(B, H, N, 32), t["wq"], t["wk"], q_block=BQ)
    with pytest.raises(ValueError):
        dsv.predict(t["q"], t["k"], t["wq"], bf(H, D, 8), q_block=BQ)
    with pytest.raises(ValueError):
        dsv.predict(t["q"], t["k"], t["wq"], t["wk"], q_block=BQ, out=f32(B, H, NQB, NKB - 1))
    with pytest.raises(ValueError):
        dsv.predict_select_representative(t["q"], t["k"], t["wq"], t["wk"], K, 0, q_block=BQ, out=i32(B, H, NQB, K + 1))
    with pytest.raises(ValueError):
        dsv.select_topk(f32(B, H, NQB, NKB), K, q_block=BQ, out=i32(B, H, NQB, K - 1))
    with pytest.raises(ValueError):
        dsv.select_mass(f32(B, H, NQB, NKB), 0.5, K, q_block=BQ, out=(i32(B, H, NQB, K), i32(B, H, NQB + 1)))
    with pytest.raises(ValueError):
        dsv.block_recall(f32(B, H, N), f32(B, H, N - 64), q_block=BQ)
    with pytest.raises(ValueError):
        dsv.block_recall(f32(B, H, N), f32(B, H, N), q_block=BQ, out=f32(B, H, NQB - 1))
    with pytest.raises(ValueError):
        dsv.pack_kv(t["k"], bf(B, H, N, 32), t["idx"], 0, 1, q_block=BQ)
