"""Peak-rate probes on the device: each returns a positive rate in the range the chip allows.

The bounds are deliberately wide (they are not a performance test): the MI355X vendor peaks are
2.5 PFLOP/s dense bf16/fp16 MFMA, an exponential rate of 256 CUs x 4 SIMDs x 8 lanes x 2.4 GHz
(half the non-packed fp32 FMA rate) and 8 TB/s of HBM; a correct probe lands below each and
well above a small fraction of it.
"""
import pytest
import torch

import dynamic_sparse_attention_dsv_amd as dsv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,lo,hi", [("mfma_bf16", 0.5e15, 2.6e15), ("mfma_f16", 0.5e15, 2.6e15),
                                        ("exp_f32", 4e12, 2.0e13), ("hbm_copy", 1.5e12, 8.2e12),
                                        ("hbm_read", 1.5e12, 8.2e12)])
def test_peak_probe_rates_are_plausible(kind, lo, hi):
    rate = dsv.peak_probe(kind, repeats=3)
    torch.cuda.synchronize()
    print(f"[probe] {kind}: {rate:.4g}", flush=True)
    assert lo < rate < hi, (kind, rate)
