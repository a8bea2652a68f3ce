"""Host-side checks of the C ABI: the library loads, exports every function the
header declares with C linkage, its struct layout matches the header, and
invalid arguments are rejected on the host before any device work."""
import ctypes
import os
import re
import subprocess

import pytest

import dynamic_sparse_attention_dsv_amd as dsv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsv.LIB_PATH):
        pytest.skip("libdsv.so not built")
    return dsv.load_library()


def test_every_declared_function_is_exported(lib):
    declared = _declared_functions()
    assert len(declared) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", dsv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    assert sorted(dsv.EXPORTED) == declared


def test_problem_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "dsv.h"\n'
                   "int main(void){printf(\"%zu %zu %zu %zu\\n\", sizeof(dsv_problem), "
                   "offsetof(dsv_problem, dtype), offsetof(dsv_problem, sm_scale), offsetof(dsv_problem, pred_scale));"
                   "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    size, off_dtype, off_sm, off_ps = map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                                              check=True).stdout.split())
    assert size == ctypes.sizeof(dsv.Problem)
    assert off_dtype == dsv.Problem.dtype.offset
    assert off_sm == dsv.Problem.sm_scale.offset and off_ps == dsv.Problem.pred_scale.offset


def test_status_strings_and_version(lib):
    for code, name in dsv.STATUS.items():
        assert lib.dsv_status_string(code).decode() == name
    assert lib.dsv_version() >= 100


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails validation first


def _prob(**kw):
    base = dict(batch=1, heads=2, seq_len=1024, head_dim=64, q_block=64, kv_block=64, topk=2, rank=16,
                dtype=dsv.DSV_BF16, sm_scale=0.0, pred_scale=0.0)
    base.update(kw)
    return dsv.Problem(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(topk=0), 1), (dict(topk=17), 1), (dict(seq_len=1000), 1), (dict(q_block=96), 1),
    (dict(batch=0), 1), (dict(dtype=7), 1), (dict(head_dim=96), 2), (dict(kv_block=32, q_block=64), 2),
    (dict(seq_len=64 * 5000, q_block=64, kv_block=64), 2),
])
def test_forward_rejects_bad_problems_before_launch(lib, kw, code):
    p = _prob(**kw)
    st = lib.dsv_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == code, lib.dsv_last_error()
    assert lib.dsv_last_error().decode()


def test_null_and_misaligned_pointers_are_rejected(lib):
    p = _prob()
    assert lib.dsv_select_topk(None, FAKE, FAKE, None) == 1
    assert lib.dsv_select_topk(ctypes.byref(p), None, FAKE, None) == 1
    assert lib.dsv_select_topk(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 2), FAKE, None) == 1
    assert "aligned" in lib.dsv_last_error().decode()
    st = lib.dsv_sparse_attn_fwd(ctypes.byref(p), FAKE, ctypes.c_void_p((1 << 20) + 8), FAKE, FAKE, None, FAKE, FAKE,
                                 None, FAKE, 1 << 40, None)
    assert st == 1
    st = lib.dsv_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 2), FAKE, FAKE,
                                 None, FAKE, 1 << 40, None)
    assert st == 1 and "block_counts" in lib.dsv_last_error().decode()


def test_o_residual_is_bf16_only_and_aligned(lib):
    args = lambda prob, olo: (ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, olo, FAKE, 1 << 40, None)
    p32 = _prob(dtype=dsv.DSV_F32)
    assert lib.dsv_sparse_attn_fwd(*args(p32, FAKE)) == 1
    assert "o_lo" in lib.dsv_last_error().decode()
    assert lib.dsv_sparse_attn_fwd(*args(_prob(), ctypes.c_void_p((1 << 20) + 4))) == 1
    assert "o_lo" in lib.dsv_last_error().decode()
    nb = lib.dsv_sparse_attn_bwd_workspace_size(ctypes.byref(p32))
    st = lib.dsv_sparse_attn_bwd(ctypes.byref(p32), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                 FAKE, FAKE, nb, None)
    assert st == 1 and "o_lo" in lib.dsv_last_error().decode()


def test_predict_workspace_is_the_projections_then_two_mass_halves_per_score_slot(lib):
    # bf16: Q~ and K_lr ([B, H, N, r] bf16 each), then per persistent score workgroup two
    # [N/64][256] float halves of per-row block masses (one filled by the sweep while the other
    # waits for its finalisation).  2 heads x 1024 rows / 256 make eight work items, so eight
    # workgroups on any device with two or more compute units.
    p = _prob()
    lr = 1 * 2 * 1024 * 16 * 2
    slots, nkb = 2 * 1024 // 256, 1024 // 64
    nw = lib.dsv_predict_workspace_size(ctypes.byref(p))
    assert nw == 2 * lr + slots * 2 * nkb * 256 * 4
    assert lib.dsv_predict(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, nw - 1, FAKE, None) == 3
    assert "workspace" in lib.dsv_last_error().decode()


def test_workspace_sizes_and_short_workspace_is_rejected(lib):
    p = _prob()
    # bf16 training forward (o_lo given): an fp16 copy of V, B*H*N*d*2 bytes, plus per-head words
    nf = lib.dsv_sparse_attn_fwd_workspace_size(ctypes.byref(p))
    assert nf >= 2 * 1024 * 64 * 2
    assert lib.dsv_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, nf - 1,
                                   None) == 3
    assert "workspace" in lib.dsv_last_error().decode()
    assert lib.dsv_sparse_attn_fwd_workspace_size(ctypes.byref(_prob(dtype=dsv.DSV_F32))) == 0
    nb = lib.dsv_sparse_attn_bwd_workspace_size(ctypes.byref(p))
    # bf16 backward: lse2 + D (2 x B*H*N floats), the block-order list, and the transposed block lists
    assert nb >= 2 * 2 * 1024 * 4 + 2 * 16 * 4 + 2 * 16 * 2 * 4
    st = lib.dsv_sparse_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                 FAKE, FAKE, nb - 1, None)
    assert st == 3
    assert lib.dsv_sparse_attn_fwd_workspace_size(None) == 0
    assert lib.dsv_sparse_attn_bwd_workspace_size(None) == 0


def test_predictor_rejects_unsupported_rank(lib):
    p = _prob(rank=24)
    st = lib.dsv_predict(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, FAKE, None)
    assert st == 2
    p = _prob(seq_len=64 * 3, q_block=64)  # N % 256 != 0 for the bf16 predictor
    p.topk = 1
    assert lib.dsv_predict(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, FAKE, None) == 2


def test_select_mass_validates_tau_and_pointers(lib):
    p = _prob(topk=4)
    for tau in (0.0, -0.5, 1.5, float("nan")):
        assert lib.dsv_select_mass(ctypes.byref(p), FAKE, ctypes.c_float(tau), FAKE, FAKE, None) == 1
        assert "tau" in lib.dsv_last_error().decode()
    assert lib.dsv_select_mass(ctypes.byref(p), FAKE, ctypes.c_float(0.9), FAKE, None, None) == 1
    assert "block_counts" in lib.dsv_last_error().decode()
    assert lib.dsv_select_mass(ctypes.byref(_prob(topk=17)), FAKE, ctypes.c_float(0.9), FAKE, FAKE, None) == 1


def test_representative_predictor_validates_the_row(lib):
    p = _prob()
    for rep in (-1, 64):
        assert lib.dsv_predict_representative(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, rep, FAKE, 1 << 40, FAKE,
                                              None) == 1
        assert "rep_row" in lib.dsv_last_error().decode()


def test_pack_validates_range_and_workspace(lib):
    p = _prob(topk=4)
    nb = lib.dsv_pack_kv_workspace_size(ctypes.byref(p))
    assert nb >= 2 * 2 * 16 * 4
    args = lambda b, e, ws: (ctypes.byref(p), FAKE, FAKE, FAKE, None, b, e, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    for b, e in ((-1, 2), (3, 2), (0, 17)):
        assert lib.dsv_pack_kv(*args(b, e, nb)) == 1
        assert "qb_begin" in lib.dsv_last_error().decode()
    assert lib.dsv_pack_kv(*args(0, 4, nb - 1)) == 3


def test_block_recall_validates_pointers(lib):
    p = _prob()
    assert lib.dsv_block_recall(ctypes.byref(p), FAKE, None, FAKE, None) == 1
    assert "lse_all" in lib.dsv_last_error().decode()
    assert lib.dsv_block_recall(None, FAKE, FAKE, FAKE, None) == 1


def test_bf16_backward_rejects_extreme_softmax_scales(lib):
    for sc in (2.0 ** 50, 2.0 ** -50):
        p = _prob(sm_scale=sc)
        nb = lib.dsv_sparse_attn_bwd_workspace_size(ctypes.byref(p))
        st = lib.dsv_sparse_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                     FAKE, FAKE, nb, None)
        assert st == 2 and "sm_scale" in lib.dsv_last_error().decode()


def test_head_density_validates_threshold(lib):
    p = _prob()
    for thr in (-0.1, float("nan"), float("inf")):
        assert lib.dsv_head_density(ctypes.byref(p), None, ctypes.c_float(thr), FAKE, None, None) == 1
        assert "dense_above" in lib.dsv_last_error().decode()
    assert lib.dsv_head_density(ctypes.byref(p), None, ctypes.c_float(0.5), None, None, None) == 1


def test_native_caller_is_built_and_checks_its_arguments():
    exe = os.path.join(ROOT, "tests", "native", "abi_roundtrip")
    if not os.path.exists(exe):
        pytest.skip("native caller not built")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    r = subprocess.run([exe, "/nonexistent", "/tmp/x", "1", "1", "1024", "64", "16", "64", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 1 and "cannot read" in r.stderr


def test_peak_probe_validates_before_any_launch(lib):
    # workspace sizes: one float per probe thread (MFMA, exp), 1 GiB for the copy; 0 = unknown kind
    assert lib.dsv_peak_probe_workspace_size(0) == lib.dsv_peak_probe_workspace_size(2) > 0
    assert lib.dsv_peak_probe_workspace_size(3) == 1 << 30
    assert lib.dsv_peak_probe_workspace_size(4) > 1 << 30
    assert lib.dsv_peak_probe_workspace_size(5) == 0 and lib.dsv_peak_probe_workspace_size(-1) == 0
    rate = ctypes.c_double(0.0)
    nb = lib.dsv_peak_probe_workspace_size(0)
    assert lib.dsv_peak_probe(9, 1, FAKE, nb, ctypes.byref(rate), None) == 1          # unknown kind
    assert lib.dsv_peak_probe(0, 0, FAKE, nb, ctypes.byref(rate), None) == 1          # repeats out of range
    assert lib.dsv_peak_probe(0, 101, FAKE, nb, ctypes.byref(rate), None) == 1
    assert lib.dsv_peak_probe(0, 1, FAKE, nb, None, None) == 1                        # no rate pointer
    assert lib.dsv_peak_probe(0, 1, None, nb, ctypes.byref(rate), None) == 1          # no workspace
    assert lib.dsv_peak_probe(0, 1, ctypes.c_void_p((1 << 20) + 16), nb, ctypes.byref(rate), None) == 1  # alignment
    assert lib.dsv_peak_probe(3, 1, FAKE, (1 << 30) - 1, ctypes.byref(rate), None) == 3  # workspace too small
    assert "workspace" in lib.dsv_last_error().decode()
    assert rate.value == 0.0


def test_noalloc_pack_rejects_problems_beyond_its_scratch(lib):
    # B*H*N/Bk = 65 * 4096 entries exceeds the library's 262144-entry device array: refused on the
    # host before any launch, with the limit named
    p = _prob(heads=65, seq_len=262144, head_dim=128, q_block=128, topk=8)
    st = lib.dsv_pack_kv_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, None, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == 2 and "allocation-free limit" in lib.dsv_last_error().decode()
    # exactly at the limit the size passes and the pointer checks run
    p = _prob(heads=64, seq_len=262144, head_dim=128, q_block=128, topk=8)
    st = lib.dsv_pack_kv_noalloc(ctypes.byref(p), FAKE, FAKE, None, None, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == 1 and "block_idx" in lib.dsv_last_error().decode()
