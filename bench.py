#!/usr/bin/env python3
"""Benchmark of one DSV attention-layer step on one MI355X.

A step is the whole hot path over one batch of synthetic video tokens:
predict (low-rank block scores) -> select (top-k KV blocks) -> sparse attention
forward -> sparse attention backward, all in the HIP library.  The default
workload is the long-video layer: B=1, H=40, N=131072 (32x64x64 latent), d=128,
r=32, 128-token query blocks, 64-token KV blocks, k=205 of 2048 (10% density).

Prints ONE JSON line.  `value` is the effective sparse-attention throughput of
the whole step: forward+backward attention flops (4*B*H*N*k*Bk*d, times 3.5)
divided by the full step time, predictor and selection included.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C5]
                       [--no-dense] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (vendor figure)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E peak (vendor figure)
# Transcendental (v_exp_f32) peak: 256 CUs x 4 SIMDs x 8 lanes per cycle (half the non-packed fp32 FMA
# rate, 16 lanes per SIMD per cycle) x 2.4 GHz.  The predictor needs one exponential per logit.
EXP_PEAK_T = 256 * 4 * 8 * 2.4e9 / 1e12


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="C5")
    ap.add_argument("--generator", choices=("g1", "g2"), default=None,
                    help="override the config's input generator (g2: smooth Q field and 3D-cube token order)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense (k = N/Bk) comparator")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the oracle sample")
    ap.add_argument("--no-mass", action="store_true", help="skip the mass-threshold selection leg")
    ap.add_argument("--no-rep", action="store_true", help="skip the representative-row predictor leg")
    ap.add_argument("--no-pack", action="store_true", help="skip the KV-packing (sequence-sharding) leg")
    ap.add_argument("--mass-tau", type=float, default=0.1,
                    help="tau of the mass-threshold leg (kmax = 2k); with the random-init predictor's near-uniform "
                         "scores, 0.1 selects about the headline density")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the measured-peak probes (MFMA bf16/fp16, exp, HBM copy)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (a reference for HBM byte counters)")
    return ap.parse_args()


def kernel_units(cfg):
    """Algorithmic work per launch of each kernel, and the roofline it is judged against."""
    pairs = cfg.batch * cfg.heads * cfg.nqb * cfg.topk          # selected (query block, KV block) pairs
    unit = cfg.q_block * cfg.kv_block * cfg.head_dim              # Bq*Bk*d
    elems = cfg.batch * cfg.heads * cfg.seq_len * cfg.head_dim
    return {
        # forward: S = Q K^T and O = P V over every selected pair
        "attn_fwd_kernel": ("mfma", 4.0 * pairs * unit),
        # backward, 10*Bq*Bk*d per pair: S, dP, dV, dK (8 units) in the KV-parallel kernel,
        # dQ (2 units) in the query-parallel kernel (its S and dP are recomputation)
        "attn_bwd_dkdv_kernel": ("mfma", 8.0 * pairs * unit),
        "attn_bwd_dq_kernel": ("mfma", 2.0 * pairs * unit),
        # predictor sweep: one exponential per predicted logit, B*H*N^2 of them
        "scores_kernel": ("alu", float(cfg.batch * cfg.heads) * cfg.seq_len * cfg.seq_len),
        "select_topk_kernel": ("hbm", 4.0 * cfg.batch * cfg.heads * cfg.nqb * (cfg.nkb + cfg.topk)),
        "select_mass_kernel": ("hbm", 4.0 * cfg.batch * cfg.heads * cfg.nqb * (cfg.nkb + min(2 * cfg.topk, cfg.nkb) + 1)),
        # projection of one tensor: read [B,H,N,d] bf16, write [B,H,N,r] bf16
        "proj_kernel(q)": ("hbm", 2.0 * elems + 2.0 * cfg.batch * cfg.heads * cfg.seq_len * cfg.rank),
        "bwd_pre_kernel": ("hbm", 2.0 * 2 * elems + 12.0 * cfg.batch * cfg.heads * cfg.seq_len),
    }


def measured_traffic(cfg, timing_name):
    """HBM bytes per launch (read + write) of a kernel from the committed counter summary of this
    workload, or None when there is none or the kernel's sources changed since it was taken."""
    from dynamic_sparse_attention_dsv_amd.profile_summary import source_hash

    path = os.path.join(ROOT, "profiles", f"{cfg.name.lower()}_kernel_traffic.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as fh:
        summary = json.load(fh)
    # counters of another input generator (another selection) do not describe this run
    if not summary.get("workload", "").endswith(f"{cfg.generator} inputs"):
        return None, None
    rec = summary.get("kernels", {}).get(timing_name)
    if rec is None or rec.get("source_sha256") != source_hash(timing_name):
        return None, None
    return rec["read_bytes"] + rec["write_bytes"], os.path.relpath(path, ROOT)


def cpu_baseline(cfg, inp, target_s):
    """The CPU oracle on a bounded sample of the same workload (one head, the first query blocks)."""
    from threadpoolctl import threadpool_limits

    from oracle import dsv_oracle as O
    from workloads.generator import widen

    cores = len(os.sched_getaffinity(0))
    sc = 1.0 / np.sqrt(cfg.head_dim)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        xq, xk, xv, xdo = (widen(inp[n][0, 0]) for n in ("q", "k", "v", "do"))
        qlr = O.project_query(xq, widen(inp["wq"][0]), sc, cfg.dtype)
        klr = O.project(xk, widen(inp["wk"][0]), cfg.dtype)
        done = 0
        while True:
            rows = slice(done * cfg.q_block, (done + 1) * cfg.q_block)
            s = O.block_scores_qblock(qlr[rows], klr, cfg.kv_block, O.LN2)
            idx = O.select_topk_row(s, cfg.topk)
            O.attn_fwd_qblock(xq[rows], xk, xv, idx, cfg.kv_block, sc)
            O.attn_bwd_qblock(xq[rows], xk, xv, xdo[rows], idx, cfg.kv_block, sc)
            done += 1
            if time.perf_counter() - t0 >= target_s or done >= cfg.nqb:
                break
        dt = time.perf_counter() - t0
    flops = 14.0 * done * cfg.q_block * cfg.topk * cfg.kv_block * cfg.head_dim
    # heads and query blocks are independent, so the whole layer scales linearly from the sample
    layer_s = dt / done * cfg.nqb * cfg.heads * cfg.batch
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"head 0 of {cfg.name}, {done} of {cfg.nqb} query blocks: projections, full-key predictor "
                      f"sweep, top-k, sparse forward and backward in float64 NumPy ({dt:.1f} s)",
            "seconds": dt, "query_blocks": done,
            "extrapolated_layer_s": layer_s,
            "extrapolated_layer_note": f"one full layer ({cfg.batch * cfg.heads} heads x {cfg.nqb} query blocks) "
                                       "at the sample's rate, extrapolated (linear in heads and query blocks)"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}): the library has no multi-GPU path; "
              "its sharding design is documented with it", file=sys.stderr)
        sys.exit(2)
    import torch

    import dynamic_sparse_attention_dsv_amd as dsv
    from workloads import get_config, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dsv.load_library()
    cfg = get_config(a.config)
    if a.generator:
        cfg = cfg.with_(generator=a.generator)
    dev = torch.device("cuda:0")
    log(f"[bench] {cfg.name}: B={cfg.batch} H={cfg.heads} N={cfg.seq_len} d={cfg.head_dim} r={cfg.rank} "
        f"Bq={cfg.q_block} Bk={cfg.kv_block} k={cfg.topk}/{cfg.nkb}; generating inputs")
    t0 = time.perf_counter()
    inp = make_inputs(cfg, with_grad=True, workers=min(16, len(os.sched_getaffinity(0))))
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")

    def to_dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    t = {k: to_dev(v) for k, v in inp.items()}
    B, H, N, D = t["q"].shape
    kw = dict(q_block=cfg.q_block, kv_block=cfg.kv_block)
    ws_p, ws_f, ws_b = dsv.workspace_sizes(t["q"], topk=cfg.topk, rank=cfg.rank, **kw)
    wsp = torch.empty(ws_p, dtype=torch.uint8, device=dev)
    wsf = torch.empty(max(ws_f, 1), dtype=torch.uint8, device=dev)
    wsb = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    scores = torch.empty((B, H, cfg.nqb, cfg.nkb), dtype=torch.float32, device=dev)
    idx = torch.empty((B, H, cfg.nqb, cfg.topk), dtype=torch.int32, device=dev)
    o, lse = torch.empty_like(t["q"]), torch.empty((B, H, N), dtype=torch.float32, device=dev)
    o_lo = torch.empty_like(t["q"])  # the forward's O residual, handed to the backward
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    def step(marks=None):
        if marks: marks[0].record(stream)
        dsv.predict(t["q"], t["k"], t["wq"], t["wk"], workspace=wsp, out=scores, **kw)
        if marks: marks[1].record(stream)
        dsv.select_topk(scores, cfg.topk, out=idx, **kw)
        if marks: marks[2].record(stream)
        dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx, workspace=wsf, residual=True, out=(o, lse, o_lo), **kw)
        if marks: marks[3].record(stream)
        dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, idx, o_lo=o_lo, workspace=wsb, out=(dq, dk, dv),
                            **kw)
        if marks: marks[4].record(stream)

    if a.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB read + 1 GiB written by one copy kernel")
        del src, dst
    for i in range(a.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{a.warmup} done")
    phases = np.zeros(4)
    dsv.timing_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(ev)
        ev[4].synchronize()
        phases += [ev[j].elapsed_time(ev[j + 1]) for j in range(4)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kstats = dsv.timing_end()
    ms_step = wall * 1e3 / a.steps
    phases /= a.steps
    log(f"[bench] {a.steps} steps: {ms_step:.2f} ms/step (predict {phases[0]:.2f}, select {phases[1]:.2f}, "
        f"fwd {phases[2]:.2f}, bwd {phases[3]:.2f} ms)")

    attn_flops = cfg.fwd_flops() + cfg.bwd_flops()
    value = attn_flops / (ms_step * 1e-3) / 1e12
    attn_ms = phases[2] + phases[3]
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    kern = {n: {"launches": s[0], "avg_ms": s[1] / s[0], "min_ms": s[2], "max_ms": s[3]} for n, s in kstats.items()}

    # roofline of the dominant kernel (largest total time)
    units = kernel_units(cfg)
    dom = max(kstats, key=lambda n: kstats[n][1])
    bound, work = units.get(dom, ("unknown", None))
    avg_s = kstats[dom][1] / kstats[dom][0] * 1e-3
    roof = {"kernel": dom, "avg_ms": avg_s * 1e3}
    if bound == "mfma":
        ach = work / avg_s / 1e12
        roof.update(bound="mfma", achieved=ach, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=ach / MFMA_BF16_PEAK_TFLOPS, traffic=None)
    elif bound == "hbm":
        ach = work / avg_s / 1e9
        roof.update(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s", frac=ach / HBM_PEAK_GBS, traffic=None)
    elif bound == "alu":
        ach = work / avg_s / 1e12
        roof.update(bound="alu", achieved=ach, peak=EXP_PEAK_T, unit="Texp/s", frac=ach / EXP_PEAK_T, traffic=None)
    else:
        roof.update(bound=bound, achieved=None, peak=None, unit=None, frac=None, traffic=None)
    roof["traffic"], roof["traffic_source"] = measured_traffic(cfg, dom)
    # per-kernel rates for the attention kernels
    rates = {}
    peaks = {"mfma": (MFMA_BF16_PEAK_TFLOPS, 1e12, "TFLOP/s"), "hbm": (HBM_PEAK_GBS, 1e9, "GB/s"),
             "alu": (EXP_PEAK_T, 1e12, "Texp/s")}
    for n, (bnd, work) in units.items():
        if n in kstats and work:
            s = kstats[n][1] / kstats[n][0] * 1e-3
            pk, scale, unit = peaks[bnd]
            rates[n] = {"bound": bnd, "achieved": work / s / scale, "unit": unit, "frac": work / s / scale / pk}

    # measured peaks (after the timed region): the rates this device sustains for the bounding
    # operations, beside the vendor figures
    measured = None
    if not a.no_probe:
        log("[bench] measured peaks (MFMA bf16/fp16, exp, HBM copy probes)")
        measured = {"mfma_bf16_tflops": dsv.peak_probe("mfma_bf16") / 1e12,
                    "mfma_f16_tflops": dsv.peak_probe("mfma_f16") / 1e12,
                    "exp_texp_per_s": dsv.peak_probe("exp_f32") / 1e12,
                    "hbm_copy_gbs": dsv.peak_probe("hbm_copy") / 1e9,
                    "hbm_read_gbs": dsv.peak_probe("hbm_read") / 1e9}
        log(f"[bench] measured peaks: {measured}")
        mpk = {"mfma": measured["mfma_bf16_tflops"], "alu": measured["exp_texp_per_s"], "hbm": measured["hbm_read_gbs"]}
        for r in list(rates.values()) + [roof]:
            if r.get("achieved") is not None and r.get("bound") in mpk:
                r["peak_measured"] = mpk[r["bound"]]
                r["frac_measured"] = r["achieved"] / mpk[r["bound"]]

    dense = None
    if not a.no_dense:
        log("[bench] dense comparator (k = N/Bk through the same kernels)")
        idx_d = torch.arange(cfg.nkb, dtype=torch.int32, device=dev).repeat(B, H, cfg.nqb, 1).contiguous()
        _, wsf_d, wsb_d = dsv.workspace_sizes(t["q"], topk=cfg.nkb, rank=cfg.rank, **kw)
        wsb2 = torch.empty(wsb_d, dtype=torch.uint8, device=dev)
        del wsb
        lse_sel = lse.clone()  # the top-k step's lse, for the recall of its selection
        dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx_d, workspace=wsf, residual=True, out=(o, lse, o_lo), **kw)
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx_d, workspace=wsf, residual=True, out=(o, lse, o_lo), **kw)
        e1.record(stream)
        dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, idx_d, o_lo=o_lo, workspace=wsb2,
                            out=(dq, dk, dv), **kw)
        e2.record(stream)
        e2.synchronize()
        dfwd, dbwd = e0.elapsed_time(e1), e1.elapsed_time(e2)
        dense_flops = 3.5 * 4.0 * B * H * N * N * D
        # the dense forward's lse (every block selected) gives the true mass the top-k lists capture
        dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx_d, workspace=wsf, residual=True, out=(o, lse, o_lo), **kw)
        rec = dsv.block_recall(lse_sel, lse, q_block=cfg.q_block).double()
        torch.cuda.synchronize()
        dense = {"fwd_ms": dfwd, "bwd_ms": dbwd, "tflops": dense_flops / ((dfwd + dbwd) * 1e-3) / 1e12,
                 "speedup_attn": (dfwd + dbwd) / attn_ms, "ideal_speedup": cfg.nkb / cfg.topk,
                 "recall_mean": float(rec.mean()), "recall_p05": float(torch.quantile(rec.flatten()[:1 << 24], 0.05)),
                 "recall_min": float(rec.min())}
        log(f"[bench] dense fwd {dfwd:.1f} ms bwd {dbwd:.1f} ms; top-k recall mean {dense['recall_mean']:.4f} "
            f"p05 {dense['recall_p05']:.4f} min {dense['recall_min']:.4f}")

    mass = None
    if not a.no_mass:
        # mass-threshold selection and attention over the resulting ragged lists, same inputs
        kmax = min(2 * cfg.topk, cfg.nkb)
        log(f"[bench] mass-threshold leg (tau={a.mass_tau}, kmax={kmax})")
        idx_m = torch.empty((B, H, cfg.nqb, kmax), dtype=torch.int32, device=dev)
        cnt_m = torch.empty((B, H, cfg.nqb), dtype=torch.int32, device=dev)
        _, _, wsb_m = dsv.workspace_sizes(t["q"], topk=kmax, rank=cfg.rank, **kw)
        wsb3 = torch.empty(wsb_m, dtype=torch.uint8, device=dev)
        dsv.predict(t["q"], t["k"], t["wq"], t["wk"], workspace=wsp, out=scores, **kw)
        evm = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for rep in range(2):  # the first pass warms up
            evm[0].record(stream)
            dsv.select_mass(scores, a.mass_tau, kmax, out=(idx_m, cnt_m), **kw)
            evm[1].record(stream)
            dsv.sparse_attn_fwd(t["q"], t["k"], t["v"], idx_m, block_counts=cnt_m, workspace=wsf, residual=True,
                                out=(o, lse, o_lo), **kw)
            evm[2].record(stream)
            dsv.sparse_attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, idx_m, block_counts=cnt_m, o_lo=o_lo,
                                workspace=wsb3, out=(dq, dk, dv), **kw)
            evm[3].record(stream)
            evm[3].synchronize()
        ms = [evm[j].elapsed_time(evm[j + 1]) for j in range(3)]
        pairs_m = int(cnt_m.sum().item())
        flops_m = 14.0 * pairs_m * cfg.q_block * cfg.kv_block * cfg.head_dim
        # per-head activation: selected density, and heads whose density exceeds one half
        dens, dflag = dsv.head_density(cnt_m, topk=kmax, seq_len=N, q_block=cfg.q_block, kv_block=cfg.kv_block,
                                       dense_above=0.5)
        mass = {"tau": a.mass_tau, "kmax": kmax, "mean_count": pairs_m / (B * H * cfg.nqb),
                "min_count": int(cnt_m.min().item()), "max_count": int(cnt_m.max().item()),
                "head_density_min": float(dens.min()), "head_density_max": float(dens.max()),
                "heads_dense_above_half": int(dflag.sum()),
                "select_ms": ms[0], "fwd_ms": ms[1], "bwd_ms": ms[2],
                "attn_tflops": flops_m / ((ms[1] + ms[2]) * 1e-3) / 1e12}
        log(f"[bench] mass leg: mean count {mass['mean_count']:.1f}, select {ms[0]:.2f} ms, fwd {ms[1]:.1f} ms, "
            f"bwd {ms[2]:.1f} ms")
        del wsb3

    rep = None
    if not a.no_rep:
        # representative-row predictor (one row per query block) and top-k on its scores
        log("[bench] representative-row leg (row 0 of each query block)")
        evr = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for _ in range(2):  # the first pass warms up
            evr[0].record(stream)
            dsv.predict(t["q"], t["k"], t["wq"], t["wk"], rep_row=0, workspace=wsp, out=scores, **kw)
            evr[1].record(stream)
            dsv.select_topk(scores, cfg.topk, out=idx, **kw)
            evr[2].record(stream)
            evr[2].synchronize()
        rep = {"rep_row": 0, "predict_ms": evr[0].elapsed_time(evr[1]), "select_ms": evr[1].elapsed_time(evr[2]),
               "logits": float(B * H * cfg.nqb) * N}
        # the fused predictor + top-k (indices straight from the projections, no score matrix)
        idx_f = torch.empty_like(idx)
        for _ in range(2):  # the first pass warms up
            evr[0].record(stream)
            dsv.predict_select_representative(t["q"], t["k"], t["wq"], t["wk"], cfg.topk, 0, workspace=wsp,
                                              out=idx_f, **kw)
            evr[1].record(stream)
            evr[1].synchronize()
        rep["fused_ms"] = evr[0].elapsed_time(evr[1])
        rep["fused_equal_to_unfused"] = float((idx_f == idx).all(dim=-1).float().mean())
        log(f"[bench] representative leg: predict {rep['predict_ms']:.2f} ms, select {rep['select_ms']:.2f} ms; "
            f"fused {rep['fused_ms']:.2f} ms (rows equal to the unfused pair: {rep['fused_equal_to_unfused']:.4f})")

    pack = None
    if not a.no_pack:
        # KV packing for one eighth of the query blocks (one GPU's share under 8-way sequence
        # sharding), with the top-k lists of the timed steps
        qb1 = cfg.nqb // 8
        log(f"[bench] KV packing leg (query blocks [0, {qb1}))")
        evp = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(2):  # the first pass warms up
            evp[0].record(stream)
            kp, vp, pblocks, pcounts, _ = dsv.pack_kv(t["k"], t["v"], idx, 0, qb1, **kw)
            evp[1].record(stream)
            evp[1].synchronize()
        ms_p = evp[0].elapsed_time(evp[1])
        units = int(pcounts.sum().item())
        moved = 2.0 * 2 * units * cfg.kv_block * D * t["k"].element_size()  # K and V, read + write
        pack = {"query_blocks": qb1, "mean_union_blocks": units / (B * H), "ms": ms_p, "bytes_moved": moved,
                "gbs": moved / (ms_p * 1e-3) / 1e9}
        log(f"[bench] pack leg: union {pack['mean_union_blocks']:.0f} of {cfg.nkb} blocks per head, {ms_p:.2f} ms, "
            f"{pack['gbs']:.0f} GB/s")
        del kp, vp

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] CPU oracle baseline (bounded sample)")
        cpu = cpu_baseline(cfg, inp, a.cpu_seconds)

    rec = {
        "metric": "sparse attn fwd+bwd effective TFLOP/s & tokens/s at N=131k, 10% density",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (seeded smooth-bias video-token generator, random-init predictor)",
        "config": {"workload": f"{cfg.name}: long-video attention layer, B={B} H={H} latent "
                               f"{'x'.join(map(str, cfg.latent))} N={N} d={D} r={cfg.rank} Bq={cfg.q_block} "
                               f"Bk={cfg.kv_block} top-{cfg.topk} of {cfg.nkb} KV blocks",
                   "batch": B, "heads": H, "seq_len": N, "head_dim": D, "rank": cfg.rank, "q_block": cfg.q_block,
                   "kv_block": cfg.kv_block, "topk": cfg.topk, "density": cfg.topk / cfg.nkb,
                   "generator": cfg.generator},
        "tokens_per_s": B * N / (ms_step * 1e-3),
        "attn_fwd_bwd": {"ms": attn_ms, "tflops": attn_tflops, "frac_of_peak": attn_tflops / MFMA_BF16_PEAK_TFLOPS,
                         "frac_of_measured_peak": attn_tflops / measured["mfma_bf16_tflops"] if measured else None,
                         "tokens_per_s": B * N / (attn_ms * 1e-3)},
        "measured_peaks": measured,
        "phases_ms": {"predict": phases[0], "select": phases[1], "fwd": phases[2], "bwd": phases[3]},
        "kernels": kern, "kernel_rates": rates, "dense": dense, "mass_selection": mass, "representative": rep, "pack": pack,
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
