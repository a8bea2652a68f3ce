"""bench.py without a GPU: its one-GPU contract and the algorithmic work its rates divide by."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_config  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr


# (config, forward flops, forward + backward flops, predicted logits B*H*N^2), as tabulated for the
# workloads from 4*B*H*N*(k*Bk)*d, the backward at 2.5x the forward, and one logit per (row, key)
WORK = [("C1", 67.1e6, 234.9e6, 2.1e6), ("C2", 20.9e9, 73.3e9, 0.81e9), ("C3", 335.0e9, 1.17e12, 6.44e9),
        ("C4", 8.85e12, 30.97e12, 171.8e9), ("C4b", 4.38e12, 15.33e12, 171.8e9),
        ("C5", 35.22e12, 123.27e12, 687.2e9)]


@pytest.mark.parametrize("name,fwd,total,logits", WORK)
def test_algorithmic_work_matches_the_tabulated_figures(name, fwd, total, logits):
    cfg = get_config(name)
    assert cfg.fwd_flops() == pytest.approx(fwd, rel=6e-3)
    assert cfg.fwd_flops() + cfg.bwd_flops() == pytest.approx(total, rel=6e-3)
    units = bench.kernel_units(cfg)
    # the three attention kernels are credited exactly the method's 14 Bq*Bk*d per selected pair
    credited = sum(units[k][1] for k in ("attn_fwd_kernel", "attn_bwd_dkdv_kernel", "attn_bwd_dq_kernel"))
    assert credited == pytest.approx(cfg.fwd_flops() + cfg.bwd_flops(), rel=1e-12)
    assert units["attn_fwd_kernel"][1] == pytest.approx(cfg.fwd_flops(), rel=1e-12)
    assert units["scores_kernel"] == ("alu", pytest.approx(logits, rel=6e-3))
